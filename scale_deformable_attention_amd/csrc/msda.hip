// msda.hip -- gfx950 kernels and the C ABI of the multi-scale deformable
// attention core (declared in include/msda.h).
//
// What is computed: for every (batch b, query q, head m), the sum over levels l
// and points k of A[b,q,m,l,k] times the bilinear sample of level l, head m at
// the location phi_l(loc) = (u*W_l - 0.5, v*H_l - 0.5), pixels outside the
// level reading as zero (MSDeformAttn equation of the deformable-attention
// tutorial, discosf.com section 2.2; cell-centre grid_sample semantics of the
// cf-1.com fallback, section 5.3), and the gradients of that sum (discosf.com
// section 3.2).
//
// Work mapping (one kernel design for every supported D and value type):
//  * a "tuple" is one (b, q, m); its D channels are one contiguous row of the
//    value tensor per pixel, so a group of G = D*sizeof(T)/16 lanes covers a
//    row with one 16-byte load per lane, and a 64-lane wave runs 64/G tuples
//    side by side;
//  * per chunk, every lane first computes the sampling record of ONE point
//    (coordinate map, cell, the four corner offsets and weights), so the
//    scalar-like work is done once per point instead of once per lane, and
//    parks it in the wave's slice of LDS;
//  * each group then reads the records of its own tuple (LDS broadcast) and
//    issues the four corner-row loads as raw buffer loads. A corner outside
//    the level gets an offset past the buffer's record count, which the
//    hardware answers with zeros: no branch, no clamp, no out-of-range access;
//  * the backward reduces the four per-corner dot products g.v_c across the
//    group with DPP, and the record's owner lane turns them into the weight
//    and location gradients; grad_value is scattered with fp32 buffer atomics
//    (also dropped by the hardware for outside corners).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "msda.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
// Byte offset given to corners outside their level: past the record count of
// every buffer the kernels build (all are smaller than 2 GiB), also after the
// bf16 -> fp32 doubling of the backward's grad_value offsets.
constexpr uint32_t kOutside = 0xC0000000u;
// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
    uint16_t bits;
};

// Reinterpret bits as fp32. Takes the word by value on purpose: this compiler
// miscompiles __builtin_bit_cast applied directly to an element of an
// ext_vector_type value (it reads element 0 whatever the index).
__device__ inline float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kPerLane = 4;  // 16 bytes per lane
    static constexpr int kBytes = 4;
    __device__ static inline void widen(u32x4 raw, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = as_float(raw[i]);
    }
};
template <>
struct Elem<bf16_t> {
    static constexpr int kPerLane = 8;
    static constexpr int kBytes = 2;
    // bf16 is the top half of an fp32: widening is exact.
    __device__ static inline void widen(u32x4 raw, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = as_float(raw[i] << 16);
            v[2 * i + 1] = as_float(raw[i] & 0xFFFF0000u);
        }
    }
};

template <typename T, int D>
struct Shape {
    static constexpr int kPerLane = Elem<T>::kPerLane;
    static constexpr int G = D / kPerLane;   // lanes per tuple
    static constexpr int TPW = kWave / G;    // tuples per wave
    static_assert(G >= 1 && G <= 16 && (G & (G - 1)) == 0, "unsupported D for this type");
};

struct Params {
    const void* value;
    const int64_t* shapes;
    const int64_t* lsi;
    const float* loc;
    const float* attn;
    float* out;
    const float* grad_out;
    float* grad_value;
    float* grad_loc;
    float* grad_attn;
    int Nv, M, L, Nq, K, LK;
    int T;                    // tuples B*Nq*M
    uint32_t value_bytes;     // record count of the value buffer
    uint32_t grad_value_bytes;
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferWord3);
}

__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the G consecutive lanes of a group (G a power of two <= 16); every
// lane of the group receives the sum. Butterfly: xor 1, xor 2 (quad
// permutations), then the mirrors within 8 and 16 lanes.
template <int G>
__device__ inline float group_sum(float v) {
    if constexpr (G >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (G >= 16) v += dpp<0x140>(v); // row_mirror
    return v;
}

// Level table (H, W, start row) staged once per block.
__device__ inline void load_levels(const Params& p, int4* levels) {
    if (threadIdx.x < (unsigned)p.L) {
        const int l = threadIdx.x;
        levels[l] = make_int4((int)p.shapes[2 * l], (int)p.shapes[2 * l + 1], (int)p.lsi[l], 0);
    }
    __syncthreads();
}

// Sampling geometry of one point: cell, fractions, validity of the four
// corners (0: (y0,x0), 1: (y0,x0+1), 2: (y0+1,x0), 3: (y0+1,x0+1)) and the
// corner rows' byte offsets relative to the tuple's base.
struct Geometry {
    float fx, fy;
    bool valid[4];
    uint32_t off[4];
};

__device__ inline Geometry point_geometry(float u, float v, int4 lv, uint32_t tuple_base,
                                          uint32_t row_bytes) {
    Geometry g;
    const float Hf = (float)lv.x, Wf = (float)lv.y;
    // cell-centre map, one rounding (the oracle uses the same fp32 fma)
    const float x = fmaf(u, Wf, -0.5f);
    const float y = fmaf(v, Hf, -0.5f);
    const float x0f = floorf(x), y0f = floorf(y);
    g.fx = x - x0f;
    g.fy = y - y0f;
    // bounds tests written so that NaN fails them
    const bool vx0 = (x0f >= 0.0f) && (x0f < Wf);
    const bool vx1 = (x0f >= -1.0f) && (x0f < Wf - 1.0f);
    const bool vy0 = (y0f >= 0.0f) && (y0f < Hf);
    const bool vy1 = (y0f >= -1.0f) && (y0f < Hf - 1.0f);
    g.valid[0] = vx0 && vy0;
    g.valid[1] = vx1 && vy0;
    g.valid[2] = vx0 && vy1;
    g.valid[3] = vx1 && vy1;
    // clamp before converting so that the integer math below is defined for
    // any input; the clamped value is only used for valid corners
    const int x0 = (int)fminf(fmaxf(x0f, -1.0f), Wf);
    const int y0 = (int)fminf(fmaxf(y0f, -1.0f), Hf);
    const int row00 = lv.z + y0 * lv.y + x0;
    const uint32_t o00 = tuple_base + (uint32_t)row00 * row_bytes;
    g.off[0] = g.valid[0] ? o00 : kOutside;
    g.off[1] = g.valid[1] ? o00 + row_bytes : kOutside;
    g.off[2] = g.valid[2] ? o00 + (uint32_t)lv.y * row_bytes : kOutside;
    g.off[3] = g.valid[3] ? o00 + (uint32_t)(lv.y + 1) * row_bytes : kOutside;
    return g;
}

// Byte offset, within the value tensor, of tuple t's row 0: (b*Nv*M + m)*D*elem.
__device__ inline uint32_t tuple_base_bytes(const Params& p, int t, int row_bytes, int head_bytes) {
    const int b = t / (p.Nq * p.M);
    const int m = t - (t / p.M) * p.M;
    return (uint32_t)b * (uint32_t)p.Nv * (uint32_t)row_bytes + (uint32_t)m * (uint32_t)head_bytes;
}

// ------------------------------------------------------------------ forward
struct FwdRecord {
    uint32_t off[4];
    float w[4];   // A * bilinear weight, 0 for corners outside
};

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void msda_fwd_kernel(Params p) {
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW, PL = S::kPerLane;
    constexpr int kRowBytesPerHead = D * Elem<T>::kBytes;
    __shared__ int4 levels[MSDA_MAX_LEVELS];
    __shared__ FwdRecord records[kWavesPerBlock][kWave];
    load_levels(p, levels);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int tuple0 = (blockIdx.x * kWavesPerBlock + wave) * TPW;
    if (tuple0 >= p.T) return;  // wave-uniform; no block barrier follows
    const uint32_t row_bytes = (uint32_t)p.M * kRowBytesPerHead;
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.value, p.value_bytes);

    // phase-1 role: this lane builds records of tuple t1 = tuple0 + lane % TPW
    const int t1 = tuple0 + lane % TPW;
    const int jrow = lane / TPW;
    const bool t1_ok = t1 < p.T;
    const uint32_t base1 = t1_ok ? tuple_base_bytes(p, t1, row_bytes, kRowBytesPerHead) : 0;
    // phase-2 role: this lane accumulates channels [r*PL, r*PL+PL) of tuple t2
    const int g = lane / G, r = lane % G;
    const int t2 = tuple0 + g;

    float acc[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] = 0.0f;

    for (int jc = 0; jc < p.LK; jc += G) {
        // phase 1: one point per lane -> record in LDS
        FwdRecord rec;
        const int j = jc + jrow;
        if (t1_ok && j < p.LK) {
            const int l = (unsigned)j / (unsigned)p.K;
            const int4 lv = levels[l];
            const size_t pt = (size_t)t1 * p.LK + j;
            const float2 uv = *reinterpret_cast<const float2*>(p.loc + 2 * pt);
            const float a = p.attn[pt];
            const Geometry geo = point_geometry(uv.x, uv.y, lv, base1, row_bytes);
            const float ay0 = a * (1.0f - geo.fy), ay1 = a * geo.fy;
            const float w[4] = {ay0 * (1.0f - geo.fx), ay0 * geo.fx, ay1 * (1.0f - geo.fx),
                                ay1 * geo.fx};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rec.off[c] = geo.off[c];
                rec.w[c] = geo.valid[c] ? w[c] : 0.0f;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rec.off[c] = kOutside;
                rec.w[c] = 0.0f;
            }
        }
        records[wave][lane] = rec;
        wave_sync();
        // phase 2: the group gathers its G points of this chunk
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const FwdRecord q = records[wave][i * TPW + g];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(
                    vrsrc, q.off[c] + (uint32_t)r * 16u, 0, 0);
                float v[PL];
                Elem<T>::widen(raw, v);
#pragma unroll
                for (int e = 0; e < PL; ++e) acc[e] = fmaf(q.w[c], v[e], acc[e]);
            }
        }
        wave_sync();
    }
    if (t2 < p.T) {
        float4* dst = reinterpret_cast<float4*>(p.out + (size_t)t2 * D + r * PL);
#pragma unroll
        for (int e = 0; e < PL; e += 4) dst[e / 4] = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
}

// ------------------------------------------------------------------ backward
struct BwdRecord {
    uint32_t off[4];
    float aw[4];  // A * bilinear weight, 0 for corners outside
    float dot[4]; // sum_d g[d] * v_c[d], filled by the gathering group
};

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void msda_bwd_kernel(Params p) {
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW, PL = S::kPerLane;
    constexpr int kRowBytesPerHead = D * Elem<T>::kBytes;
    // grad_value is fp32: its byte offsets are the value offsets times this
    constexpr int kGradScale = 4 / Elem<T>::kBytes;
    __shared__ int4 levels[MSDA_MAX_LEVELS];
    __shared__ BwdRecord records[kWavesPerBlock][kWave];
    load_levels(p, levels);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int tuple0 = (blockIdx.x * kWavesPerBlock + wave) * TPW;
    if (tuple0 >= p.T) return;
    const uint32_t row_bytes = (uint32_t)p.M * kRowBytesPerHead;
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.value, p.value_bytes);
    const __amdgpu_buffer_rsrc_t grsrc =
        make_rsrc(p.grad_value, p.grad_value ? p.grad_value_bytes : 0u);

    const int t1 = tuple0 + lane % TPW;
    const int jrow = lane / TPW;
    const bool t1_ok = t1 < p.T;
    const uint32_t base1 = t1_ok ? tuple_base_bytes(p, t1, row_bytes, kRowBytesPerHead) : 0;
    const int g = lane / G, r = lane % G;
    const int t2 = tuple0 + g;

    // upstream gradient of the group's tuple, this lane's channels
    float go[PL];
    if (t2 < p.T) {
        const float4* src = reinterpret_cast<const float4*>(p.grad_out + (size_t)t2 * D + r * PL);
#pragma unroll
        for (int e = 0; e < PL; e += 4) {
            const float4 v4 = src[e / 4];
            go[e] = v4.x;
            go[e + 1] = v4.y;
            go[e + 2] = v4.z;
            go[e + 3] = v4.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < PL; ++e) go[e] = 0.0f;
    }

    for (int jc = 0; jc < p.LK; jc += G) {
        // phase 1: this lane's point -> record; keep what phase 3 needs
        const int j = jc + jrow;
        const bool mine = t1_ok && j < p.LK;
        size_t pt = 0;
        float a = 0.0f, Hf = 0.0f, Wf = 0.0f;
        Geometry geo;
        BwdRecord rec;
        if (mine) {
            const int l = (unsigned)j / (unsigned)p.K;
            const int4 lv = levels[l];
            pt = (size_t)t1 * p.LK + j;
            const float2 uv = *reinterpret_cast<const float2*>(p.loc + 2 * pt);
            a = p.attn[pt];
            Hf = (float)lv.x;
            Wf = (float)lv.y;
            geo = point_geometry(uv.x, uv.y, lv, base1, row_bytes);
            const float ay0 = a * (1.0f - geo.fy), ay1 = a * geo.fy;
            const float w[4] = {ay0 * (1.0f - geo.fx), ay0 * geo.fx, ay1 * (1.0f - geo.fx),
                                ay1 * geo.fx};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rec.off[c] = geo.off[c];
                rec.aw[c] = geo.valid[c] ? w[c] : 0.0f;
                rec.dot[c] = 0.0f;
            }
        } else {
            geo.fx = geo.fy = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                geo.valid[c] = false;
                geo.off[c] = kOutside;
                rec.off[c] = kOutside;
                rec.aw[c] = 0.0f;
                rec.dot[c] = 0.0f;
            }
        }
        records[wave][lane] = rec;
        wave_sync();
        // phase 2: gather, per-corner dot products, grad_value scatter
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int slot = i * TPW + g;
            const uint32_t off[4] = {records[wave][slot].off[0], records[wave][slot].off[1],
                                     records[wave][slot].off[2], records[wave][slot].off[3]};
            const float aw[4] = {records[wave][slot].aw[0], records[wave][slot].aw[1],
                                 records[wave][slot].aw[2], records[wave][slot].aw[3]};
            float dot[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 raw = __builtin_amdgcn_raw_buffer_load_b128(
                    vrsrc, off[c] + (uint32_t)r * 16u, 0, 0);
                float v[PL];
                Elem<T>::widen(raw, v);
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < PL; ++e) s = fmaf(go[e], v[e], s);
                dot[c] = s;
                if (p.grad_value) {
                    const uint32_t goff = off[c] * kGradScale + (uint32_t)r * (PL * 4);
#pragma unroll
                    for (int e = 0; e < PL; ++e)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(aw[c] * go[e], grsrc,
                                                                        goff + 4u * e, 0, 0);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) dot[c] = group_sum<G>(dot[c]);
            if (r == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) records[wave][slot].dot[c] = dot[c];
            }
        }
        wave_sync();
        // phase 3: the record's owner turns the four dot products into the
        // weight and location gradients of its point
        if (mine) {
            float dot[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) dot[c] = records[wave][lane].dot[c];
            const float fx = geo.fx, fy = geo.fy;
            const float w[4] = {(1.0f - fx) * (1.0f - fy), fx * (1.0f - fy), (1.0f - fx) * fy,
                                fx * fy};
            const float dwdx[4] = {-(1.0f - fy), (1.0f - fy), -fy, fy};
            const float dwdy[4] = {-(1.0f - fx), -fx, (1.0f - fx), fx};
            float ga = 0.0f, gx = 0.0f, gy = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (geo.valid[c]) {
                    ga = fmaf(w[c], dot[c], ga);
                    gx = fmaf(dwdx[c], dot[c], gx);
                    gy = fmaf(dwdy[c], dot[c], gy);
                }
            }
            if (p.grad_attn) p.grad_attn[pt] = ga;
            if (p.grad_loc)
                *reinterpret_cast<float2*>(p.grad_loc + 2 * pt) = make_float2(a * Wf * gx, a * Hf * gy);
        }
        wave_sync();
    }
}

__global__ __launch_bounds__(kBlock) void zero_fill_kernel(float4* dst, int64_t n4) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * kBlock)
        dst[i] = z;
}

// ------------------------------------------------------------------ host side
constexpr int64_t k2GiB = int64_t(1) << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b <= limit for non-negative a, b, without overflow
bool mul_le(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

// Host checks shared by both entry points. Every offset the kernels form is
// 32-bit: the value (and fp32 grad_value) tensors must stay below 2 GiB and the
// tuple count below 2^31 minus a block.
msda_status_t check_dims(const msda_dims_t* d, msda_dtype_t dt, bool backward) {
    if (!d) return MSDA_ERROR_INVALID_VALUE;
    if (d->B < 0 || d->Nq < 0 || d->K < 0 || d->M < 1 || d->Nv < 1 || d->L < 1 || d->D < 1)
        return MSDA_ERROR_INVALID_VALUE;
    if (dt != MSDA_DTYPE_F32 && dt != MSDA_DTYPE_BF16) return MSDA_ERROR_INVALID_VALUE;
    if (d->L > MSDA_MAX_LEVELS) return MSDA_ERROR_NOT_SUPPORTED;
    if (d->D != 8 && d->D != 16 && d->D != 32 && d->D != 64) return MSDA_ERROR_NOT_SUPPORTED;
    const int64_t lim = k2GiB - 1;
    const int64_t elem = (backward || dt == MSDA_DTYPE_F32) ? 4 : 2;  // widest buffer
    if (!mul_le(d->Nv, d->M, lim) || !mul_le(d->Nv * d->M, d->D * elem, lim) ||
        !mul_le(d->B, d->Nv * d->M * d->D * elem, lim))
        return MSDA_ERROR_NOT_SUPPORTED;
    if (!mul_le(d->Nq, d->M, lim) || !mul_le(d->B, d->Nq * d->M, lim - 1024))
        return MSDA_ERROR_NOT_SUPPORTED;
    if (!mul_le(d->L, d->K, lim / 2)) return MSDA_ERROR_NOT_SUPPORTED;
    return MSDA_SUCCESS;
}

Params make_params(const msda_dims_t* d, msda_dtype_t dt, const void* value, const int64_t* shapes,
                   const int64_t* lsi, const float* loc, const float* attn) {
    Params p = {};
    p.value = value;
    p.shapes = shapes;
    p.lsi = lsi;
    p.loc = loc;
    p.attn = attn;
    p.Nv = (int)d->Nv;
    p.M = (int)d->M;
    p.L = (int)d->L;
    p.Nq = (int)d->Nq;
    p.K = (int)d->K;
    p.LK = (int)(d->L * d->K);
    p.T = (int)(d->B * d->Nq * d->M);
    const int64_t elems = d->B * d->Nv * d->M * d->D;
    p.value_bytes = (uint32_t)(elems * (dt == MSDA_DTYPE_BF16 ? 2 : 4));
    p.grad_value_bytes = (uint32_t)(elems * 4);
    return p;
}

// Element counts of the tensors (for the NULL-pointer rules).
struct Sizes {
    int64_t value, points, out;
};
Sizes sizes_of(const msda_dims_t* d) {
    Sizes s;
    s.value = d->B * d->Nv * d->M * d->D;
    s.points = d->B * d->Nq * d->M * d->L * d->K;
    s.out = d->B * d->Nq * d->M * d->D;
    return s;
}

template <typename T, int D>
int tuples_per_block() {
    return Shape<T, D>::TPW * kWavesPerBlock;
}

msda_status_t launch(const void* kernel, int64_t blocks, Params& p, hipStream_t stream) {
    if (blocks <= 0) return MSDA_SUCCESS;
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3(kBlock), args, 0, stream);
    return e == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_LAUNCH;
}

template <typename T, int D>
const void* fwd_kernel() {
    return reinterpret_cast<const void*>(&msda_fwd_kernel<T, D>);
}
template <typename T, int D>
const void* bwd_kernel() {
    return reinterpret_cast<const void*>(&msda_bwd_kernel<T, D>);
}

// Picks the instantiation for (value type, D); returns its tuples per block.
template <bool kBackward>
const void* pick(msda_dtype_t dt, int64_t D, int* tpb) {
#define MSDA_PICK(T, DD)                                                          \
    if (D == DD) {                                                                \
        *tpb = tuples_per_block<T, DD>();                                         \
        return kBackward ? bwd_kernel<T, DD>() : fwd_kernel<T, DD>();             \
    }
    if (dt == MSDA_DTYPE_F32) {
        MSDA_PICK(float, 8) MSDA_PICK(float, 16) MSDA_PICK(float, 32) MSDA_PICK(float, 64)
    } else {
        MSDA_PICK(bf16_t, 8) MSDA_PICK(bf16_t, 16) MSDA_PICK(bf16_t, 32) MSDA_PICK(bf16_t, 64)
    }
#undef MSDA_PICK
    return nullptr;
}

}  // namespace

extern "C" {

msda_status_t msda_forward(const msda_dims_t* dims, msda_dtype_t value_dtype, const void* value,
                           const int64_t* spatial_shapes, const int64_t* level_start_index,
                           const float* sampling_locations, const float* attention_weights,
                           float* output, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, value_dtype, false);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(dims);
    // a tensor with no elements may come as NULL
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_locations || !attention_weights)) || (n.out && !output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(output, 16) || !aligned(sampling_locations, 8) ||
        !aligned(attention_weights, 4) || !aligned(spatial_shapes, 8) ||
        !aligned(level_start_index, 8))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, value_dtype, value, spatial_shapes, level_start_index,
                           sampling_locations, attention_weights);
    p.out = output;
    if (p.T == 0) return MSDA_SUCCESS;
    int tpb = 0;
    const void* k = pick<false>(value_dtype, dims->D, &tpb);
    if (!k) return MSDA_ERROR_NOT_SUPPORTED;
    return launch(k, ((int64_t)p.T + tpb - 1) / tpb, p, stream);
}

msda_status_t msda_backward(const msda_dims_t* dims, msda_dtype_t value_dtype, const void* value,
                            const int64_t* spatial_shapes, const int64_t* level_start_index,
                            const float* sampling_locations, const float* attention_weights,
                            const float* grad_output, float* grad_value,
                            float* grad_sampling_locations, float* grad_attention_weights,
                            hipStream_t stream) {
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(dims);
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_locations || !attention_weights)) || (n.out && !grad_output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(grad_output, 16) || !aligned(grad_value, 16) ||
        !aligned(sampling_locations, 8) || !aligned(grad_sampling_locations, 8) ||
        !aligned(attention_weights, 4) || !aligned(grad_attention_weights, 4) ||
        !aligned(spatial_shapes, 8) || !aligned(level_start_index, 8))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, value_dtype, value, spatial_shapes, level_start_index,
                           sampling_locations, attention_weights);
    p.grad_out = grad_output;
    p.grad_value = grad_value;
    p.grad_loc = grad_sampling_locations;
    p.grad_attn = grad_attention_weights;
    int tpb = 0;
    const void* k = pick<true>(value_dtype, dims->D, &tpb);
    if (!k) return MSDA_ERROR_NOT_SUPPORTED;
    if (grad_value && n.value) {
        // fill kernel rather than a memset node: safe inside captured graphs
        const int64_t n4 = n.value / 4;
        const int64_t blocks = n4 / kBlock < 4096 ? (n4 + kBlock - 1) / kBlock : 4096;
        float4* dst = reinterpret_cast<float4*>(grad_value);
        int64_t count = n4;
        void* args[] = {&dst, &count};
        if (hipLaunchKernel(reinterpret_cast<const void*>(&zero_fill_kernel),
                            dim3((unsigned)blocks), dim3(kBlock), args, 0, stream) != hipSuccess)
            return MSDA_ERROR_LAUNCH;
    }
    if (p.T == 0 || (!grad_value && !grad_sampling_locations && !grad_attention_weights))
        return MSDA_SUCCESS;
    return launch(k, ((int64_t)p.T + tpb - 1) / tpb, p, stream);
}

msda_status_t msda_check_tables(const int64_t* host_spatial_shapes,
                                const int64_t* host_level_start_index, int64_t L, int64_t Nv) {
    if (!host_spatial_shapes || !host_level_start_index || L < 1 || L > MSDA_MAX_LEVELS || Nv < 1)
        return MSDA_ERROR_INVALID_VALUE;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        const int64_t H = host_spatial_shapes[2 * l], W = host_spatial_shapes[2 * l + 1];
        if (H < 1 || W < 1 || H > k2GiB || W > k2GiB) return MSDA_ERROR_INVALID_VALUE;
        if (host_level_start_index[l] != total) return MSDA_ERROR_INVALID_VALUE;
        total += H * W;
        if (total > k2GiB) return MSDA_ERROR_INVALID_VALUE;
    }
    return total == Nv ? MSDA_SUCCESS : MSDA_ERROR_INVALID_VALUE;
}

const char* msda_status_string(msda_status_t status) {
    switch (status) {
        case MSDA_SUCCESS: return "success";
        case MSDA_ERROR_INVALID_VALUE: return "invalid value (pointer, alignment or size)";
        case MSDA_ERROR_NOT_SUPPORTED: return "not supported (D, level count or tensor size)";
        case MSDA_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int msda_version(void) {
    return MSDA_VERSION_MAJOR * 10000 + MSDA_VERSION_MINOR * 100 + MSDA_VERSION_PATCH;
}

}  // extern "C"
