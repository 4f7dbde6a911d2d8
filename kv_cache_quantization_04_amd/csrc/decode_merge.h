// Merge of the split-K partials of decode attention (gfx950): the reduce kernel's
// per-head merge, and the same merge run inside a decode kernel by the workgroup that
// finishes last among the splits of a (sequence, kv head).
#pragma once
#include "common.h"
#include "launch.h"
#include "xlane.h"

namespace kvq {

// Device-coherent accesses of the split partials: the stores write through the
// issuing XCD's L2 and the loads do not take a line from the reader's L2, so that a
// workgroup on one XCD reads, within the same kernel, what workgroups on others wrote,
// with no write-back or invalidation of whole caches (which a release / acquire fence
// at device scope performs, at a cost of microseconds per workgroup).
__device__ __forceinline__ void store_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev2(const float *p) {
    const uint64_t b = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return float2{__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}
// partial loads of the merge: COH inside the decode kernel that wrote them, plain in
// the reduce kernel (a kernel boundary orders them)
template <bool COH>
__device__ __forceinline__ float ld_part(const float *p) {
    if constexpr (COH) return load_dev(p);
    else return *p;
}
template <bool COH>
__device__ __forceinline__ float2 ld_part2(const float *p) {
    if constexpr (COH) return load_dev2(p);
    else return *reinterpret_cast<const float2 *>(p);
}

// Merge the split partials of one (sequence, query head), normalize, rotate back.
// One wave per (sequence, query head), no workgroup barriers: lane l owns the
// E = Dv / 64 consecutive channels E l .. E l + E - 1. The lanes load the split
// maxima and sums in parallel (split i on lane i mod 64), reduce them across the
// wave, and leave the weights exp(m_i - M) in a wave-private LDS array; the
// output pass then streams the partial outputs with independent loads. The
// inverse rotation runs in registers (channel bits below E) and across lanes.
constexpr int RED_MAX_SPLITS = 1024;
constexpr int RED_WAVES = 4;

__device__ __forceinline__ float wave_max(float v) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Up to RED_FAST splits with at most two channels per lane: every load in one round
// (split i's maximum and sum on lane i, all partial outputs on every lane), the
// maxima and sums reduced over the first 16 lanes with DPP row operations and read
// back as wave-uniform values; the outputs accumulate in split order, as below.
constexpr int RED_FAST = 16;

template <int E, bool COH>
__device__ __forceinline__ void reduce_weights_fast(const float *w, int S, int lane, float (&part)[RED_FAST][E],
                                                    float (&e)[RED_FAST], float &l) {
    constexpr int Dv = 64 * E;
    float mi = -INFINITY, li = 0.f;
    if (lane < S) {
        mi = ld_part<COH>(w + (int64_t)lane * (Dv + 2) + Dv);
        li = ld_part<COH>(w + (int64_t)lane * (Dv + 2) + Dv + 1);
    }
#pragma unroll
    for (int i = 0; i < RED_FAST; ++i) {
        if (i < S) {  // uniform
            const float *wi = w + (int64_t)i * (Dv + 2) + E * lane;
            if constexpr (E == 1) part[i][0] = ld_part<COH>(wi);
            else {
                const float2 v = ld_part2<COH>(wi);
                part[i][0] = v.x;
                part[i][1] = v.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) part[i][k] = 0.f;
        }
    }
    const float Mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row_max16(mi))));
    const float ei = mi == -INFINITY ? 0.f : __expf(mi - Mx);
    l = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(row_sum16(ei * li))));
#pragma unroll
    for (int i = 0; i < RED_FAST; ++i) e[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ei), i));
}

template <int E, bool COH = false>
__device__ __forceinline__ void reduce_one(const DecodeArgs &a, int s, int hq, int lane, float *wgt) {
    constexpr int Dv = 64 * E;
    const float *w = a.ws + ((int64_t)s * a.Hq + hq) * a.splits * (Dv + 2);
    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.f;
    float l = 0.f;
    if (E <= 2 && a.splits <= RED_FAST) {
        float part[RED_FAST][E], e[RED_FAST];
        reduce_weights_fast<E, COH>(w, a.splits, lane, part, e, l);
#pragma unroll
        for (int i = 0; i < RED_FAST; ++i)
            if (i < a.splits)
#pragma unroll
                for (int k = 0; k < E; ++k) acc[k] = __builtin_fmaf(e[i], part[i][k], acc[k]);
    } else {
    float M = -INFINITY;
    for (int i = lane; i < a.splits; i += 64) M = fmaxf(M, ld_part<COH>(w + (int64_t)i * (Dv + 2) + Dv));
    M = wave_max(M);
    for (int i = lane; i < a.splits; i += 64) {
        const float mi = ld_part<COH>(w + (int64_t)i * (Dv + 2) + Dv);
        const float e = mi == -INFINITY ? 0.f : __expf(mi - M);
        wgt[i] = e;
        l = __builtin_fmaf(e, ld_part<COH>(w + (int64_t)i * (Dv + 2) + Dv + 1), l);
    }
    l = wave_sum(l);  // the weights' LDS writes are ordered before the reads below (one wave)
#pragma unroll 4
    for (int i = 0; i < a.splits; ++i) {
        const float *wi = w + (int64_t)i * (Dv + 2) + E * lane;
        const float e = wgt[i];
#pragma unroll
        for (int k = 0; k < E; k += (E > 1 ? 2 : 1)) {
            if constexpr (E == 1) acc[0] = __builtin_fmaf(e, ld_part<COH>(wi), acc[0]);
            else {
                const float2 v = ld_part2<COH>(wi + k);
                acc[k] = __builtin_fmaf(e, v.x, acc[k]);
                acc[k + 1] = __builtin_fmaf(e, v.y, acc[k + 1]);
            }
        }
    }
    }
    const float invl = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] *= invl;
    // Walsh-Hadamard over blocks of vh channels: channel c = E lane + k. Two channels
    // per lane and one block of 128 (head_dim 128): the lane stages by DPP, the LDS
    // crossbar (ds_swizzle, no memory) and permlane swaps instead of LDS permutes
    if (E == 2 && a.vh == 128) {
        {
            const float x = acc[0], y = acc[E - 1];
            acc[0] = x + y;
            acc[E - 1] = x - y;
        }
        auto stage = [&](auto pv_of, int m) {
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const float pv = pv_of(acc[k]);
                acc[k] = upper ? pv - acc[k] : acc[k] + pv;
            }
        };
        stage([](float v) { return dpp<DPP_QUAD_XOR1>(v); }, 1);
        stage([](float v) { return dpp<DPP_QUAD_XOR2>(v); }, 2);
        stage([](float v) { return swz_xor<4>(v); }, 4);
        stage([](float v) { return swz_xor<8>(v); }, 8);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            float lo, hi;
            pair16(acc[k], lo, hi);
            acc[k] = (lane & 16) ? lo - hi : lo + hi;
            pair32(acc[k], lo, hi);
            acc[k] = (lane & 32) ? lo - hi : lo + hi;
        }
    } else
    for (int len = 1; len < a.vh; len <<= 1) {
        if (len < E) {
#pragma unroll
            for (int k = 0; k < E; ++k)
                if (!(k & len) && (k | len) < E) {
                    const float x = acc[k], y = acc[k | len];
                    acc[k] = x + y;
                    acc[k | len] = x - y;
                }
        } else {
            const int m = len / E;  // partner lane
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const float pv = __shfl_xor(acc[k], m, 64);
                acc[k] = upper ? pv - acc[k] : acc[k] + pv;
            }
        }
    }
    const float scl = 1.0f / sqrtf((float)a.vh);
    float *out = a.out + ((int64_t)s * a.Hq + hq) * Dv + E * lane;
#pragma unroll
    for (int k = 0; k < E; ++k) out[k] = acc[k] * scl;
}

// Arrival counters at the head of a decode workspace, one per (sequence, kv head);
// larger grids merge in the reduce kernel.
constexpr int64_t MERGE_COUNTERS = KVQ_DECODE_COUNTER_BYTES / sizeof(uint32_t);

// Called by every thread of a decode workgroup after it has written its split partial
// for query heads hk g .. hk g + g - 1 of sequence s: the workgroup that arrives last
// for (s, hk) merges all splits of those heads (one wave per head, NT threads) and
// writes the output, then puts the counter back to zero for the next call. The partials
// were written with store_dev; every wave waits until its stores have completed (at the
// device coherence point) before the arrival is counted, and the last workgroup reads
// them with load_dev after its count has returned. E = Dv / 64. `wgt`: LDS scratch of
// NT / 64 * RED_MAX_SPLITS floats that the workgroup no longer uses.
template <int NT, int E>
__device__ __forceinline__ void merge_if_last(const DecodeArgs &a, int s, int hk, float *wgt) {
    __shared__ int last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *c = a.cnt + (int64_t)s * a.Hkv + hk;
        const uint32_t before = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool l = before == (uint32_t)(a.splits - 1);
        if (l) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = l;
    }
    __syncthreads();
    if (!last) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int h = wave; h < a.grp; h += NT / 64)
        reduce_one<E, true>(a, s, hk * a.grp + h, lane, wgt + wave * RED_MAX_SPLITS);
}

}  // namespace kvq
