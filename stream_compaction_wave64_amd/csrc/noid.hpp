// noid.hpp -- building blocks of scans that never use the operator's
// identity (AcceleratedKernels.jl PR #208, description, first bullet: for
// operators with no neutral element the partial results are "Optional"):
// the operator without its identity, optional carries, their descriptors,
// and the wave scan whose lanes without a source keep their value.  Used by
// the look-back pipeline (noid.hip) and the resident pass (resident.hip).
#pragma once

#include "device.hpp"

namespace sw64 {

// The element operator without its identity.
template <class Op0>
struct NoId {
    template <class T> __device__ __forceinline__ static T apply(T a, T b) { return Op0::apply(a, b); }
};

// A value that may be absent.  The flag is as wide as the value, so the
// struct has no padding and moves through DPP and descriptors as whole words.
template <class C0>
struct Opt {
    using Flag = std::conditional_t<sizeof(C0) == 8, uint64_t, uint32_t>;
    C0 v;
    Flag has;
};

// The operator extended to absent values: absent combines as a no-op, and
// "absent" is its identity.  (The placeholder value of an absent Opt is
// never combined.)
template <class Op0>
struct OptOp {
    template <class X> __device__ __forceinline__ static X identity() { return X{}; }
    template <class X> __device__ __forceinline__ static X apply(X a, X b) {
        if (!a.has) return b;
        if (!b.has) return a;
        return X{Op0::apply(a.v, b.v), 1};
    }
};

// Descriptors of Opt carries: the plain carry's words; every published
// value is present.
template <class D0>
struct OptDesc {
    static constexpr int kWords = D0::kWords;
    template <class X>
    __device__ __forceinline__ static void publish(uint64_t *d, uint32_t epoch, uint32_t state, X value) {
        D0::publish(d, epoch, state, value.v);
    }
    __device__ __forceinline__ static void fetch(const uint64_t *d, uint64_t (&w)[kWords]) { D0::fetch(d, w); }
    template <class X>
    __device__ __forceinline__ static uint32_t decode(const uint64_t (&w)[kWords], uint32_t epoch, X &value) {
        value.has = 1;
        return D0::decode(w, epoch, value.v);
    }
    template <class X>
    __device__ __forceinline__ static uint32_t read(const uint64_t *d, uint32_t epoch, X &value) {
        uint64_t w[kWords];
        fetch(d, w);
        return decode(w, epoch, value);
    }
};

// Inclusive Kogge-Stone scan over the 64 lanes (the rounds of
// wave_scan_incl) without an identity: each round combines only in the
// lanes that have a source.
template <class Op, class T>
__device__ __forceinline__ T wave_scan_incl_noid(T x) {
    const int lane = lane_id();
    T t = dpp_mov<kRowShr1>(x, x);
    if ((lane & 15) >= 1) x = Op::apply(t, x);
    t = dpp_mov<kRowShr2>(x, x);
    if ((lane & 15) >= 2) x = Op::apply(t, x);
    t = dpp_mov<kRowShr4>(x, x);
    if ((lane & 15) >= 4) x = Op::apply(t, x);
    t = dpp_mov<kRowShr8>(x, x);
    if ((lane & 15) >= 8) x = Op::apply(t, x);
    t = dpp_mov<kRowBcast15, 0xa>(x, x);  // lane 15 of rows 0 / 2 into rows 1 / 3
    if (lane & 16) x = Op::apply(t, x);
    t = dpp_mov<kRowBcast31, 0xc>(x, x);  // lane 31 into rows 2 and 3
    if (lane >= 32) x = Op::apply(t, x);
    return x;
}

}  // namespace sw64
