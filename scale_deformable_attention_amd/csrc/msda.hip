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
//    and location gradients; grad_value is built without atomics by binning
//    the points into pixel tiles and letting one block own each tile (see the
//    backward section).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <cmath>

#include "msda.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
// Byte offset given to corners outside their level: past the record count of
// every buffer the kernels build (all are smaller than 2 GiB), also after the
// bf16 -> fp32 doubling of the backward's grad_value offsets.
constexpr uint32_t kOutside = 0xC0000000u;
// The tile kernel's eight work counters (one per XCD group) sit 256 bytes
// apart: device-scope atomics on one shared line serialize across the XCDs.
constexpr int kCounterStride = 64;
// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family GPUs.
constexpr int kBufferWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
    uint16_t bits;
};
struct f16_t {
    uint16_t bits;
};

// Reinterpret bits as fp32. Takes the word by value on purpose: this compiler
// miscompiles __builtin_bit_cast applied directly to an element of an
// ext_vector_type value (it reads element 0 whatever the index).
__device__ inline float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// IEEE binary16 in the low 16 bits -> fp32 (exact).
__device__ inline float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits & 0xFFFFu));
}

// fp32 -> bf16 bits, rounded to nearest even (NaN stays a quiet NaN).
__device__ inline uint32_t float_to_bf16_bits(float f) {
    const uint32_t u = as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A 16-byte load marked non-temporal: for data read exactly once (the bin
// entries), so that it does not push reused rows out of L2.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline float4 load_streaming(const float4* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// A 16-byte store marked non-temporal: data written once and not read again
// by this kernel (the bin kernel's slab entries, read by the tile kernel that
// follows), so that it does not displace the lines the kernel reuses.
__device__ inline void store_streaming(float4* p, float4 v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

// Cache-policy operand of the raw buffer intrinsics: non-temporal.
constexpr int kBufferNonTemporal = 2;

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

template <>
struct Elem<f16_t> {
    static constexpr int kPerLane = 8;
    static constexpr int kBytes = 2;
    __device__ static inline void widen(u32x4 raw, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = raw[i];
            v[2 * i] = half_bits_to_float(w);
            v[2 * i + 1] = half_bits_to_float(w >> 16);
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
    int B, Nv, M, L, Nq, K, LK;
    int T;                    // tuples B*Nq*M
    uint32_t value_bytes;     // record count of the value buffer
    // grad_value binning (backward only)
    int nW;                   // bin blocks per (b, m)
    int Qc;                   // queries per bin block
    int t_stride;             // rows of the tile table per (b, m): tiles + 1
    int bm0, bm_count;        // the (b, m) planes of this pass: [bm0, bm0 + bm_count)
    uint32_t slab_per_block;  // point-index capacity of one bin block's slab
    uint32_t* table;          // [bm_count][t_stride][nW] slab offset of each tile's entries
                              // (tile t's count = row t+1 - row t)
    float4* slab;             // [bm_count*nW][slab_per_block] (tuple bits, x, y, A) entries
    uint32_t* counters;       // tile work counters, one per XCD group, kCounterStride apart
    uint32_t grad_value_bytes;  // record count of the grad_value buffer (its stores are range-checked)
    int slab_streaming;       // the pass's entries exceed the L2s: write them non-temporal
    // fused front-end: locations and weights formed from the model's raw
    // outputs inside the kernels
    const float* ref;         // [B, Nq, L, 2] reference points (x, y), normalized
    const float* off;         // [B, Nq, M, L, K, 2] offsets (x, y) in level pixels
    const float* logits;      // [B, Nq, M, L*K]
    float2* smax;             // [T] max and 1/sum of each tuple's exp(logit - max)
    float* grad_off;          // [B, Nq, M, L, K, 2]
    float* grad_logits;       // [B, Nq, M, L*K]
    // grouped single-level front-end (DCNv3): point k of output pixel
    // (ho, wo) samples at (wo*stride_w - pad_w + kx*dil_w, ho*stride_h - pad_h
    // + ky*dil_h) + offset, in pixels, k = ky*kernel_w + kx; the offsets are
    // read from `off` and the modulation scalars from `attn`
    int out_W, kernel_w, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
    int lvl_H, lvl_W;         // the level table when shapes is null (one level)
    int hp;                   // heads taken together in the work order (tuple_of)
};

// Where a kernel's sampling locations and weights come from.
enum FrontEnd : int {
    kFeCore = 0,    // locations and weights given
    kFeFused = 1,   // reference point + offset / (W, H), softmax of logits
    kFeDcn = 2,     // convolution grid + pixel offset, modulation scalars given
    kFeCoreHalf = 3 // locations and weights given as IEEE binary16
};

// The inputs of point j (level l) of tuple t as loaded: its location and
// weight, or (fused front-end) the reference point, the offset in level pixels
// and the logit. Loading is kept apart from finish_point's arithmetic so that
// a chunk's loads can stay in flight while the previous chunk is gathered.
struct PointIn {
    float2 uv;    // location, or the reference point
    float2 off;   // fused: offset
    float z;      // weight, or the logit
};

// (q: the tuple's query, t / M mod Nq, where the caller knows it)
template <int FE>
__device__ inline PointIn load_point_q(const Params& p, int t, int j, int l, int q) {
    PointIn in;
    const size_t pt = (size_t)t * p.LK + j;
    if constexpr (FE == kFeDcn) {
        const int ho = q / p.out_W, wo = q - ho * p.out_W;
        const int ky = j / p.kernel_w, kx = j - ky * p.kernel_w;
        in.uv = make_float2((float)(wo * p.stride_w - p.pad_w + kx * p.dil_w),
                            (float)(ho * p.stride_h - p.pad_h + ky * p.dil_h));
        in.off = *reinterpret_cast<const float2*>(p.off + 2 * pt);
        in.z = p.attn[pt];
    } else if constexpr (FE == kFeFused) {
        const size_t bq = (size_t)(t / p.M);
        in.uv = *reinterpret_cast<const float2*>(p.ref + 2 * (bq * p.L + l));
        in.off = *reinterpret_cast<const float2*>(p.off + 2 * pt);
        in.z = p.logits[pt];
    } else if constexpr (FE == kFeCoreHalf) {
        // binary16 pairs and scalars, widened exactly
        const uint32_t xy = reinterpret_cast<const uint32_t*>(p.loc)[pt];
        in.uv = make_float2(half_bits_to_float(xy), half_bits_to_float(xy >> 16));
        in.off = make_float2(0.0f, 0.0f);
        in.z = half_bits_to_float(reinterpret_cast<const uint16_t*>(p.attn)[pt]);
    } else {
        in.uv = *reinterpret_cast<const float2*>(p.loc + 2 * pt);
        in.off = make_float2(0.0f, 0.0f);
        in.z = p.attn[pt];
    }
    return in;
}

template <int FE>
__device__ inline PointIn load_point(const Params& p, int t, int j, int l) {
    return load_point_q<FE>(p, t, j, l, FE == kFeDcn ? (t / p.M) % p.Nq : 0);
}

// Fused front-end: the location is the reference point plus the offset over
// the level's size (W for x, H for y), the quotient and the sum each rounded
// to float; the weight is exp(z - max) / sum over the tuple's L*K logits
// (zmax and inv_sum are that max and 1 / sum).
// (DCNv3: the grid point plus the offset, one fp32 addition, in pixels.)
template <int FE>
__device__ inline void finish_point(const PointIn& in, int4 lv, float zmax, float inv_sum,
                                    float2& uv, float& a) {
    if constexpr (FE == kFeDcn) {
        uv.x = in.uv.x + in.off.x;
        uv.y = in.uv.y + in.off.y;
        a = in.z;
    } else if constexpr (FE == kFeFused) {
        const float qx = in.off.x / (float)lv.y;
        const float qy = in.off.y / (float)lv.x;
        uv.x = in.uv.x + qx;
        uv.y = in.uv.y + qy;
        a = expf(in.z - zmax) * inv_sum;
    } else {
        uv = in.uv;
        a = in.z;
    }
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferWord3);
}

// A value that every lane of the block holds alike (read back from LDS after a
// barrier), taken from the first lane so that the compiler sees it as
// wave-uniform: loops bounded by it, with barriers inside, then branch on a
// scalar and no lane can leave such a loop apart from the rest of its wave.
__device__ inline int block_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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
        levels[l] = p.shapes ? make_int4((int)p.shapes[2 * l], (int)p.shapes[2 * l + 1],
                                         (int)p.lsi[l], 0)
                             : make_int4(p.lvl_H, p.lvl_W, 0, 0);
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

// (x, y) in level pixels: pixel (i, j) at x = j, y = i.
__device__ inline Geometry point_geometry_px(float x, float y, int4 lv, uint32_t tuple_base,
                                             uint32_t row_bytes) {
    Geometry g;
    const float Hf = (float)lv.x, Wf = (float)lv.y;
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

// (u, v) normalized: the cell-centre map first, one rounding each (the
// oracle uses the same fp32 fma).
__device__ inline Geometry point_geometry(float u, float v, int4 lv, uint32_t tuple_base,
                                          uint32_t row_bytes) {
    return point_geometry_px(fmaf(u, (float)lv.y, -0.5f), fmaf(v, (float)lv.x, -0.5f), lv,
                             tuple_base, row_bytes);
}

template <int FE>
__device__ inline Geometry geometry_of(float2 uv, int4 lv, uint32_t tuple_base,
                                       uint32_t row_bytes) {
    if constexpr (FE == kFeDcn) return point_geometry_px(uv.x, uv.y, lv, tuple_base, row_bytes);
    return point_geometry(uv.x, uv.y, lv, tuple_base, row_bytes);
}

// Byte offset, within the value tensor, of tuple t's row 0: (b*Nv*M + m)*D*elem.
__device__ inline uint32_t tuple_base_bytes(const Params& p, int t, int row_bytes, int head_bytes) {
    const int b = t / (p.Nq * p.M);
    const int m = t - (t / p.M) * p.M;
    return (uint32_t)b * (uint32_t)p.Nv * (uint32_t)row_bytes + (uint32_t)m * (uint32_t)head_bytes;
}

// ------------------------------------------------------------------ work order
// Workgroups are handed to the 8 XCDs round-robin (block i runs on XCD i % 8)
// and each XCD has its own L2. The tuple kernels therefore walk tuples in
// (b, m, q) order (heads sharing cache lines together, see tuple_of) and give
// each XCD one contiguous share of that order: an XCD then works through one
// (b, m) value plane at a time (2.8 MB at the 800x1333 pyramid, D = 32 fp32),
// which its 4 MB L2 holds, and consecutive queries of one head sample
// neighbouring rows.
__device__ inline int xcd_block() {
    const int blk = blockIdx.x, nblk = gridDim.x;
    const int x = blk % 8, i = blk / 8, per = nblk / 8, rem = nblk % 8;
    return x * per + (x < rem ? x : rem) + i;
}

// Position in the work order -> index of the tuple in memory order
// ((b * Nq + q) * M + m). The work order is (b, m, q), except that heads whose
// rows share a 128-byte cache line (p.hp > 1 of them: rows narrower than a
// line, e.g. 64-byte bf16 rows at D = 32) are taken together, q by q:
// (b, m / hp, q, m % hp). The plane of one head alone then touches every line
// of its head group, and visiting the hp planes one after another would bring
// each line in hp times.
__device__ inline int tuple_of(const Params& p, int logical) {
    const int mi = logical % p.hp;
    const int rest = logical / p.hp;
    const int bmg = rest / p.Nq;
    const int q = rest - bmg * p.Nq;
    const int groups = p.M / p.hp;
    const int b = bmg / groups;
    const int m = (bmg - b * groups) * p.hp + mi;
    return (b * p.Nq + q) * p.M + m;
}

// ------------------------------------------------------------------ forward
struct alignas(16) FwdRecord {
    uint32_t off[4];
    float w[4];   // A * bilinear weight, 0 for corners outside
};

// A wave's LDS in the forward: the records of a chunk, or (fused front-end,
// before a round's first chunk) the partial softmax statistics.
union FwdWaveLds {
    FwdRecord records[kWave];
    float stat[kWave];
};

// ---- coarse levels in LDS
// The tuple kernels are bound by the texture path (its address and
// data-return units ~90% busy on the 800x1333 training batch), whose cost
// follows the corner gathers issued through it, by the cache lines they
// touch. Corners read from LDS do not use it. The staged forward runs a block
// over kStagedQueries queries of one (b, m) plane: the block first copies the
// rows of the plane's coarsest levels that fit in kStageBytes into LDS (at
// D = 32 fp32 on the 800x1333 pyramid: the 13 x 21 level, 35 KB), then reads
// those levels' corners there and the other levels' through buffer loads.
// The stage is kept small so that three blocks (24 waves) share a CU: stages
// of two levels and more, at one or two blocks per CU, lost more to latency
// than the texture path gained, and staging half rows (two blocks per tuple,
// one per channel half) doubled the lines each gather touches. The point
// kernel keeps the plain work order: at 16 waves per CU (its registers) the
// same staging made it slower.
constexpr int kStagedWaves = 8;
constexpr int kStagedBlock = kWave * kStagedWaves;
constexpr int kStageBytes = 36 * 1024;     // staged rows, after one zero row at offset 0
constexpr int kStagedQueries = 128;        // queries of one plane per block
constexpr int kStagedMinQueries = 2048;    // planes with fewer queries take the plain kernels

// Row widths (one head, bytes) with staged kernels.
constexpr bool staged_row(int row_bytes) { return row_bytes == 64 || row_bytes == 128; }

// Picks the coarsest levels whose rows (kRowBytes each: one head of the
// plane) fit in the stage after a zero row, and copies them from the value
// tensor (head_base: byte offset of the plane's row 0; row_stride: bytes from
// one row of the tensor to the next). stage_base[l] = byte offset of level l's
// first row in the stage, or -1. Ends with a block barrier.
template <int kRowBytes>
__device__ inline void stage_levels(const Params& p, const int4* levels, int* stage_base,
                                    unsigned char* stage, __amdgpu_buffer_rsrc_t vrsrc,
                                    uint32_t head_base, uint32_t row_stride) {
    constexpr int kPieces = kRowBytes / 16;
    static_assert(kRowBytes % 16 == 0 && kPieces <= kStagedBlock, "rows of 16-byte pieces");
    if (threadIdx.x == 0) {
        uint32_t used = kRowBytes;
        for (int l = p.L - 1; l >= 0; --l) {
            const uint64_t bytes = (uint64_t)levels[l].x * (uint64_t)levels[l].y * kRowBytes;
            if (used + bytes <= (uint64_t)kStageBytes) {
                stage_base[l] = (int)used;
                used += (uint32_t)bytes;
            } else {
                stage_base[l] = -1;
            }
        }
    }
    if (threadIdx.x < (unsigned)kPieces)
        *reinterpret_cast<u32x4*>(stage + threadIdx.x * 16u) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int l = 0; l < p.L; ++l) {
        const int sb = block_uniform(stage_base[l]);
        if (sb < 0) continue;
        // a staged level holds at most kStageBytes / kRowBytes pixels
        const int pieces = levels[l].x * levels[l].y * kPieces;
        const uint32_t src0 = head_base + (uint32_t)levels[l].z * row_stride;
        for (int i = threadIdx.x; i < pieces; i += kStagedBlock) {
            const int pix = i / kPieces, c = i - pix * kPieces;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                vrsrc, src0 + (uint32_t)pix * row_stride + (uint32_t)c * 16u, 0, 0);
            *reinterpret_cast<u32x4*>(stage + sb + i * 16) = v;
        }
    }
    __syncthreads();
}

// Whether a staged level holds point j's corners (j below LK; read from LDS,
// the same for every lane that asks about the same point).
__device__ inline bool point_staged(const Params& p, const int* stage_base, int j) {
    return stage_base[(unsigned)j / (unsigned)p.K] >= 0;
}

// One round of a forward kernel: a wave computes TPW tuples.
//  phase 1: lane (jrow, i) builds the records of points jrow, jrow + G, ... of
//           tuple t1 (one point per chunk of G), in LDS;
//  phase 2: lane group g gathers the chunk's points of tuple t2 and
//           accumulates channels [r*PL, r*PL + PL) (r: lane within the group).
// base1: byte offset of tuple t1's row 0 in the value tensor. kStaged: the
// corners of staged levels (stage_base as stage_levels left it) come from the
// stage, their outside corners from its zero row.
template <typename T, int D, int FE, bool kStaged>
__device__ __forceinline__ void fwd_round(const Params& p, const int4* levels, FwdWaveLds& wl,
                                          __amdgpu_buffer_rsrc_t vrsrc,
                                          const unsigned char* stage, const int* stage_base,
                                          int t1, bool t1_ok, uint32_t base1, int t2, bool t2_ok) {
    constexpr bool kFused = FE == kFeFused;
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW, PL = S::kPerLane;
    constexpr uint32_t kHeadBytes = D * Elem<T>::kBytes;
    const int lane = threadIdx.x & (kWave - 1);
    const int jrow = lane / TPW;
    const int g = lane / G, r = lane % G;
    const uint32_t row_bytes = (uint32_t)p.M * kHeadBytes;

    float acc[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] = 0.0f;

    // this lane's point of the next chunk is loaded one chunk ahead, while
    // the current chunk's rows are gathered
    auto fetch = [&](int jc) {
        const int j = min(jc + jrow, p.LK - 1);
        return load_point<FE>(p, t1, j, (unsigned)j / (unsigned)p.K);
    };
    PointIn in_next{};
    if (t1_ok && p.LK > 0) in_next = fetch(0);

    // fused: the softmax statistics of tuple t1 (while the first chunk's loads
    // are in flight). Its G builder lanes (lane t1 % TPW + i * TPW) each scan
    // every G-th logit, the first kZ of them kept in registers, and combine
    // through LDS.
    float zmax = 0.0f, inv_sum = 0.0f;
    if constexpr (kFused) {
        constexpr int kZ = 4;
        const float* z = p.logits + (size_t)t1 * p.LK;
        float zr[kZ];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < kZ; ++i) {
            const int j = jrow + i * G;
            zr[i] = (t1_ok && j < p.LK) ? z[j] : -INFINITY;
            mx = fmaxf(mx, zr[i]);
        }
        if (t1_ok)
            for (int j = jrow + kZ * G; j < p.LK; j += G) mx = fmaxf(mx, z[j]);
        wl.stat[lane] = mx;
        wave_sync();
        mx = -INFINITY;
        for (int i = 0; i < G; ++i) mx = fmaxf(mx, wl.stat[i * TPW + lane % TPW]);
        wave_sync();
        float se = 0.0f;
#pragma unroll
        for (int i = 0; i < kZ; ++i)
            if (t1_ok && jrow + i * G < p.LK) se += expf(zr[i] - mx);
        if (t1_ok)
            for (int j = jrow + kZ * G; j < p.LK; j += G) se += expf(z[j] - mx);
        wl.stat[lane] = se;
        wave_sync();
        se = 0.0f;
        for (int i = 0; i < G; ++i) se += wl.stat[i * TPW + lane % TPW];
        wave_sync();   // the records below reuse the statistics' LDS
        zmax = mx;
        inv_sum = 1.0f / se;
    }

    for (int jc = 0; jc < p.LK; jc += G) {
        const PointIn in = in_next;
        if (t1_ok && jc + G < p.LK) in_next = fetch(jc + G);
        // phase 1: one point per lane -> record in LDS
        FwdRecord rec;
        const int j = jc + jrow;
        bool st = false;
        if constexpr (kStaged) st = j < p.LK && point_staged(p, stage_base, j);
        if (t1_ok && j < p.LK) {
            const int l = (unsigned)j / (unsigned)p.K;
            const int4 lv = levels[l];
            float2 uv;
            float a;
            finish_point<FE>(in, lv, zmax, inv_sum, uv, a);
            const Geometry geo =
                st ? geometry_of<FE>(uv, lv, (uint32_t)stage_base[l] - (uint32_t)lv.z * kHeadBytes,
                                     kHeadBytes)
                   : geometry_of<FE>(uv, lv, base1, row_bytes);
            const float ay0 = a * (1.0f - geo.fy), ay1 = a * geo.fy;
            const float w[4] = {ay0 * (1.0f - geo.fx), ay0 * geo.fx, ay1 * (1.0f - geo.fx),
                                ay1 * geo.fx};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rec.off[c] = (st && !geo.valid[c]) ? 0u : geo.off[c];
                rec.w[c] = geo.valid[c] ? w[c] : 0.0f;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                rec.off[c] = st ? 0u : kOutside;
                rec.w[c] = 0.0f;
            }
        }
        wl.records[lane] = rec;
        wave_sync();
        // phase 2: the group gathers its G points of this chunk; point jc + i
        // lies on one level for every group, so the choice of source is
        // wave-uniform
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const FwdRecord q = wl.records[i * TPW + g];
            bool lds = false;
            if constexpr (kStaged)
                lds = block_uniform((jc + i < p.LK && point_staged(p, stage_base, jc + i)) ? 1 : 0);
            if (lds) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 raw =
                        *reinterpret_cast<const u32x4*>(stage + q.off[c] + (uint32_t)r * 16u);
                    float v[PL];
                    Elem<T>::widen(raw, v);
#pragma unroll
                    for (int e = 0; e < PL; ++e) acc[e] = fmaf(q.w[c], v[e], acc[e]);
                }
            } else {
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
        }
        wave_sync();   // the next chunk (or round) rewrites this LDS
    }
    if (t2_ok) {
        float4* dst = reinterpret_cast<float4*>(p.out + (size_t)t2 * D + r * PL);
#pragma unroll
        // non-temporal: the output is not read again here (bf16 1920x1080
        // forward 375 -> 359 us; fp32 workloads unchanged)
        for (int e = 0; e < PL; e += 4)
            store_streaming(dst + e / 4, make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]));
    }
}

// The forward over the work order: a wave takes TPW consecutive tuples.
template <typename T, int D, int FE>
__global__ __launch_bounds__(kBlock) void msda_fwd_kernel(Params p) {
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW;
    constexpr int kHeadBytes = D * Elem<T>::kBytes;
    __shared__ int4 levels[MSDA_MAX_LEVELS];
    __shared__ FwdWaveLds wave_lds[kWavesPerBlock];
    load_levels(p, levels);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int tuple0 = (xcd_block() * kWavesPerBlock + wave) * TPW;   // work-order position
    if (tuple0 >= p.T) return;  // wave-uniform; no block barrier follows
    const uint32_t row_bytes = (uint32_t)p.M * kHeadBytes;
    const int t1w = tuple0 + lane % TPW;
    const bool t1_ok = t1w < p.T;
    const int t1 = t1_ok ? tuple_of(p, t1w) : 0;
    const uint32_t base1 = t1_ok ? tuple_base_bytes(p, t1, row_bytes, kHeadBytes) : 0;
    const int t2w = tuple0 + lane / G;
    const bool t2_ok = t2w < p.T;
    const int t2 = t2_ok ? tuple_of(p, t2w) : 0;
    fwd_round<T, D, FE, false>(p, levels, wave_lds[wave], make_rsrc(p.value, p.value_bytes),
                               nullptr, nullptr, t1, t1_ok, base1, t2, t2_ok);
}

// The forward with the coarse levels in LDS: a block takes kStagedQueries
// queries of one (b, m) plane (XCD-contiguous, so that an XCD works through
// a plane at a time); its waves take rounds of TPW queries.
template <typename T, int D, int FE>
__global__ __launch_bounds__(kStagedBlock) void msda_fwd_staged_kernel(Params p) {
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW;
    constexpr int kHeadBytes = D * Elem<T>::kBytes;
    __shared__ int4 levels[MSDA_MAX_LEVELS];
    __shared__ int stage_base[MSDA_MAX_LEVELS];
    __shared__ FwdWaveLds wave_lds[kStagedWaves];
    __shared__ __align__(16) unsigned char stage[kStageBytes];
    load_levels(p, levels);

    // work item (b, m / hp, query range, m % hp): the blocks of heads whose
    // rows share cache lines (see tuple_of) take the same query range one
    // after another, on one XCD, while those lines are in its L2
    const int nqc = (p.Nq + kStagedQueries - 1) / kStagedQueries;
    const int item = xcd_block();
    const int mi = item % p.hp, rest = item / p.hp;
    const int qc = rest % nqc, bmg = rest / nqc;
    const int groups = p.M / p.hp;
    const int b = bmg / groups, m = (bmg - b * groups) * p.hp + mi;
    const int q_begin = qc * kStagedQueries, q_end = min(q_begin + kStagedQueries, p.Nq);
    const uint32_t row_bytes = (uint32_t)p.M * kHeadBytes;
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.value, p.value_bytes);
    const uint32_t head_base = (uint32_t)b * (uint32_t)p.Nv * row_bytes + (uint32_t)m * kHeadBytes;
    stage_levels<kHeadBytes>(p, levels, stage_base, stage, vrsrc, head_base, row_bytes);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // every bound of this loop is wave-uniform and no block barrier follows
    for (int q0 = q_begin + wave * TPW; q0 < q_end; q0 += kStagedWaves * TPW) {
        const int q1 = q0 + lane % TPW, q2 = q0 + lane / G;
        const bool t1_ok = q1 < q_end, t2_ok = q2 < q_end;
        const int t1 = t1_ok ? (b * p.Nq + q1) * p.M + m : 0;
        const int t2 = t2_ok ? (b * p.Nq + q2) * p.M + m : 0;
        fwd_round<T, D, FE, true>(p, levels, wave_lds[wave], vrsrc, stage, stage_base, t1, t1_ok,
                                  head_base, t2, t2_ok);
    }
}

// ------------------------------------------------------------------ backward
//
// The backward runs as up to three kernels, none of which uses a float atomic
// (on this GPU those serialize: an fp32 atomic costs a whole cache-line
// request at the memory side, and LDS fp32 atomics are slower still).
//
//  1. msda_bwd_point_kernel: the weight and location gradients. Same tuple
//     mapping as the forward; lane r of group g builds and finishes point
//     jc + r of its tuple. Per point the group gathers the four corner rows,
//     forms the four partial dot products g . v_c, reduces them across the
//     group with DPP, and the point's lane keeps them and finishes the point.
//  2. msda_bin_kernel: sorts the points into buckets by the grad_value tiles
//     (TH x TW pixels of one (b, m, level); TH = 4, or 8 where a (b, m) has
//     fewer points than pixels) their inside-the-level corners land in. A
//     block owns a range of queries of one (b, m); it counts per tile with
//     LDS integer atomics (fast), scans, writes its per-tile (count, offset)
//     row to the workspace and one 16-byte entry per (point, tile) -- tuple,
//     pixel coordinates, weight -- to its own slab (a block of at most
//     kBinUnroll points per thread loads them once, for both passes). No
//     global atomics: every block writes only its own rows.
//  3. msda_tile_kernel: persistent blocks fetch tiles from a counter per XCD
//     group. A block collects its tile's entries from every slab of the tile's
//     (b, m), sorts them by cell (counting sort in LDS, into records holding
//     the four corner weights), and lane group c sweeps cell column c - 1 top
//     to bottom, adding each entry's right corners to pixel column c and its
//     left corners to column c - 1, both in registers; the column c - 1 sums
//     then move to group c - 1 through LDS. Every grad_value element is
//     written exactly once with a plain store (zeros where nothing lands), so
//     no fill pass.
// The fused front-end adds msda_softmax_stats_kernel before these (the
// softmax max and 1/sum per tuple) and msda_ref_grad_kernel after the point
// kernel (the reference-point gradient, a sum over heads and points).

template <typename T, int D, int FE>
__global__ __launch_bounds__(kBlock) void msda_bwd_point_kernel(Params p) {
    constexpr bool kFused = FE == kFeFused;
    using S = Shape<T, D>;
    constexpr int G = S::G, TPW = S::TPW, PL = S::kPerLane;
    constexpr int kRowBytesPerHead = D * Elem<T>::kBytes;
    __shared__ int4 levels[MSDA_MAX_LEVELS];
    // corner offsets of the points of a chunk: group g's at row g (padded by
    // one slot so that the groups' broadcast reads fall in different banks)
    __shared__ uint4 offs[kWavesPerBlock][TPW][G + 1];
    load_levels(p, levels);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int tuple0 = (xcd_block() * kWavesPerBlock + wave) * TPW;   // work-order position
    if (tuple0 >= p.T) return;
    const uint32_t row_bytes = (uint32_t)p.M * kRowBytesPerHead;
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.value, p.value_bytes);

    // lane r of group g: channels [r*PL, r*PL + PL) of tuple g's rows, and
    // point jc + r of tuple g in chunk jc (built, then finished, by this lane)
    const int g = lane / G, r = lane % G;
    const int tw = tuple0 + g;
    const bool t_ok = tw < p.T;
    const int t = t_ok ? tuple_of(p, tw) : 0;
    const uint32_t base = t_ok ? tuple_base_bytes(p, t, row_bytes, kRowBytesPerHead) : 0;

    // upstream gradient of the group's tuple, this lane's channels
    float go[PL];
    if (t_ok) {
        const float4* src = reinterpret_cast<const float4*>(p.grad_out + (size_t)t * D + r * PL);
#pragma unroll
        for (int e = 0; e < PL; e += 4) {
            // read once: non-temporal where a group is eight lanes or more
            // (fp32 at D = 32: point kernel 282 -> 255 us; four-lane groups
            // measured slower)
            const float4 v4 = G >= 8 ? load_streaming(src + e / 4) : src[e / 4];
            go[e] = v4.x;
            go[e + 1] = v4.y;
            go[e + 2] = v4.z;
            go[e + 3] = v4.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < PL; ++e) go[e] = 0.0f;
    }

    // fused: the tuple's softmax statistics (computed beforehand)
    float zmax = 0.0f, inv_sum = 0.0f;
    if constexpr (kFused) {
        if (t_ok) {
            const float2 st = p.smax[t];
            zmax = st.x;
            inv_sum = st.y;
        }
    }
    float s_ag = 0.0f;   // fused: this lane's part of sum_j A_j gA_j over the tuple

    // The gradients of this lane's points are held in registers and stored
    // kHold chunks at a time (all at the end of the tuple for up to kHold
    // chunks): on this GPU loads and stores share one outstanding-operation
    // counter that drains in order, so a store issued between two chunks
    // makes every later wait for gathered rows also wait for the store's
    // acknowledgement. Slot h holds the point of chunk (first held chunk) + h:
    // xy goes to the location (or offset) gradient, s to the weight (or
    // logit, or mask) gradient. (Two slots where a lane group is 8 lanes or
    // more: four cost the fused front-end a wave per SIMD.)
    constexpr int kHold = G >= 8 ? 2 : 4;
    float2 held_xy[kHold];
    float held_s[kHold];
    float held_a[kFused ? kHold : 1];   // fused: the held points' weights A
#pragma unroll
    for (int h = 0; h < kHold; ++h) {
        held_xy[h] = make_float2(0.0f, 0.0f);
        held_s[h] = 0.0f;
        if constexpr (kFused) held_a[h] = 0.0f;
    }
    // fused, every point of the tuple held until its end: the logits'
    // gradient is finished in registers after the last chunk instead of
    // parking gA in the output and reading it back
    const bool fused_in_registers = kFused && p.LK <= kHold * G;
    auto store_held = [&](int jc0, int chunks) {
        float* xy_out = kFused || FE == kFeDcn ? p.grad_off : p.grad_loc;
        float* s_out = kFused ? p.grad_logits : p.grad_attn;
#pragma unroll
        for (int h = 0; h < kHold; ++h) {
            const int j = jc0 + h * G + r;
            if (h < chunks && t_ok && j < p.LK) {
                const size_t pt = (size_t)t * p.LK + j;
                if constexpr (kFused || FE == kFeDcn) {
                    // fused: the logits' gradient is read back below; both
                    // measured slower with non-temporal stores (DCNv3 97 ->
                    // 129 us)
                    if (xy_out) *reinterpret_cast<float2*>(xy_out + 2 * pt) = held_xy[h];
                    if (s_out) s_out[pt] = held_s[h];
                } else {
                    // written once, not read again: non-temporal, so that the
                    // L2 keeps value rows (point kernel 290 -> 279 us on the
                    // 800x1333 training batch)
                    if (xy_out)
                        __builtin_nontemporal_store(f32x2{held_xy[h].x, held_xy[h].y},
                                                    reinterpret_cast<f32x2*>(xy_out + 2 * pt));
                    if (s_out) __builtin_nontemporal_store(held_s[h], s_out + pt);
                }
            }
        }
    };

    // this lane's point of the next chunk is loaded one chunk ahead, while
    // the current chunk's rows are gathered
    auto fetch = [&](int jc) {
        const int j = min(jc + r, p.LK - 1);
        return load_point<FE>(p, t, j, (unsigned)j / (unsigned)p.K);
    };
    PointIn in_next{};
    if (t_ok && p.LK > 0) in_next = fetch(0);
    for (int jc = 0; jc < p.LK; jc += G) {
        const PointIn in = in_next;
        if (t_ok && jc + G < p.LK) in_next = fetch(jc + G);
        // phase 1: this lane's point -> corner offsets in LDS; keep the rest
        const int j = jc + r;
        const bool mine = t_ok && j < p.LK;
        float Hf = 0.0f, Wf = 0.0f;
        float a = 0.0f;
        Geometry geo;
        if (mine) {
            const int l = (unsigned)j / (unsigned)p.K;
            const int4 lv = levels[l];
            Hf = (float)lv.x;
            Wf = (float)lv.y;
            float2 uv;
            finish_point<FE>(in, lv, zmax, inv_sum, uv, a);
            geo = geometry_of<FE>(uv, lv, base, row_bytes);
        } else {
            geo.fx = geo.fy = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                geo.valid[c] = false;
                geo.off[c] = kOutside;
            }
        }
        offs[wave][g][r] = make_uint4(geo.off[0], geo.off[1], geo.off[2], geo.off[3]);
        wave_sync();
        // phase 2: the group gathers its G points and forms the per-corner dot
        // products, reduced over the group; lane i keeps those of point i
        float mine_dot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const uint4 o4 = offs[wave][g][i];
            const uint32_t off[4] = {o4.x, o4.y, o4.z, o4.w};
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
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                dot[c] = group_sum<G>(dot[c]);
                mine_dot[c] = r == i ? dot[c] : mine_dot[c];
            }
            // four-lane groups (bf16 at D = 32, fp32 at D = 16): the second half of
            // the chunk's points is scheduled after the first (DCNv3 117 -> 98 us,
            // bf16 values 229 -> 217 us; at eight-lane groups the same split
            // left the core unchanged and slowed the fused front-end)
            if constexpr (G == 4 && !kFused)
                if (i == G / 2 - 1) __builtin_amdgcn_sched_barrier(0);
        }
        wave_sync();   // the next chunk rewrites offs
        // phase 3: this lane turns the dot products into the weight and
        // location gradients of its point
        if (mine) {
            const float fx = geo.fx, fy = geo.fy;
            const float w[4] = {(1.0f - fx) * (1.0f - fy), fx * (1.0f - fy), (1.0f - fx) * fy, fx * fy};
            const float dwdx[4] = {-(1.0f - fy), (1.0f - fy), -fy, fy};
            const float dwdy[4] = {-(1.0f - fx), -fx, (1.0f - fx), fx};
            float ga = 0.0f, gx = 0.0f, gy = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (geo.valid[c]) {
                    ga = fmaf(w[c], mine_dot[c], ga);
                    gx = fmaf(dwdx[c], mine_dot[c], gx);
                    gy = fmaf(dwdy[c], mine_dot[c], gy);
                }
            }
            // fused: offsets, d loc / d off = 1 / (W, H) cancels the pixel
            // scale; the logits' gradient is finished below, once the tuple's
            // sum is known (gA parked in the output meanwhile). DCNv3: pixel
            // offsets, d(x, y) / d offset = 1, and the modulation scalar's
            // gradient is the plain weight gradient.
            const float2 xy = kFused || FE == kFeDcn ? make_float2(a * gx, a * gy)
                                                     : make_float2(a * Wf * gx, a * Hf * gy);
            const int slot = (jc / G) % kHold;
#pragma unroll
            for (int h = 0; h < kHold; ++h) {
                held_xy[h] = slot == h ? xy : held_xy[h];
                held_s[h] = slot == h ? ga : held_s[h];
                if constexpr (kFused) held_a[h] = slot == h ? a : held_a[h];
            }
            if constexpr (kFused) s_ag = fmaf(a, ga, s_ag);
        }
        // wave-uniform: every kHold-th chunk, and the last
        const int chunk = jc / G;
        if (!fused_in_registers && (chunk % kHold == kHold - 1 || jc + G >= p.LK))
            store_held(jc - (chunk % kHold) * G, chunk % kHold + 1);
    }
    if constexpr (kFused) {
        // softmax Jacobian: dL/dz_j = A_j (gA_j - sum_i A_i gA_i)
        const float s_all = group_sum<G>(s_ag);
        if (fused_in_registers) {
#pragma unroll
            for (int h = 0; h < kHold; ++h) {
                const int j = h * G + r;
                if (t_ok && j < p.LK) {
                    const size_t pt = (size_t)t * p.LK + j;
                    if (p.grad_off) *reinterpret_cast<float2*>(p.grad_off + 2 * pt) = held_xy[h];
                    if (p.grad_logits) p.grad_logits[pt] = held_a[h] * (held_s[h] - s_all);
                }
            }
        } else if (p.grad_logits && t_ok) {
            for (int j = r; j < p.LK; j += G) {
                const size_t pt = (size_t)t * p.LK + j;
                const float a = expf(p.logits[pt] - zmax) * inv_sum;
                p.grad_logits[pt] = a * (p.grad_logits[pt] - s_all);
            }
        }
    }
}

// ---- grad_value tiles
// Pixel rows per tile: kTileH, or kTileHTall where the points are sparse
// (fewer than one per pixel): a tall tile gathers twice the pixels' entries
// per work item, and with few entries per tile the per-item latency (work
// counter, table row, entry loads) is what costs.
constexpr int kTileH = 4;
constexpr int kTileHTall = 8;
constexpr int kBinRange = 1024;     // tile counters a bin block keeps in LDS at once
constexpr int kBinUnroll = 8;       // points per thread in flight in the bin kernel
constexpr int kChunk = 1024;        // entries a tile block sorts in LDS at once
constexpr int kMinQueries = 64;     // queries per bin block at least (when there are enough)
constexpr int kMaxSlabs = 256;      // bin blocks per (b, m) at most (a power of two)
constexpr int kBinSlabs = 64;       // the same unless the points then fit in registers
constexpr int kUnroll = 8;          // entries in flight per lane group in the sweep
constexpr int kUnrollTall = 2;      // the same for tall tiles (few entries per cell column)

// A tile is TH x TW pixels. Its pixels are fed by the cells (top-left
// corners) in cell rows -1 .. TH-1 and cell columns -1 .. TW-1 relative to
// it: NG = TW + 1 cell columns, one per lane group of a tile block (4 fp32
// channels per lane).
template <int D, int TH>
struct TileShape {
    static constexpr int PL = 4;
    static constexpr int G = D / PL;
    static constexpr int NG = kBlock / G;   // lane groups
    static constexpr int TW = NG - 1;       // pixel columns per tile
    static constexpr int kCells = (TH + 1) * NG;
    static_assert(TW >= 15, "tile width");
};

struct LevelTiles {
    int H, W, start, tile_base, ntx, pad0, pad1, pad2;
};

// Per-level tile grid of one (b, m): thread 0 fills the table, everyone waits.
template <int TW, int TH>
__device__ inline void setup_tiles(const Params& p, LevelTiles* lt, int* total) {
    if (threadIdx.x == 0) {
        int base = 0;
        for (int l = 0; l < p.L; ++l) {
            LevelTiles t;
            t.H = p.shapes ? (int)p.shapes[2 * l] : p.lvl_H;
            t.W = p.shapes ? (int)p.shapes[2 * l + 1] : p.lvl_W;
            t.start = p.shapes ? (int)p.lsi[l] : 0;
            t.tile_base = base;
            t.ntx = (t.W + TW - 1) / TW;
            t.pad0 = t.pad1 = t.pad2 = 0;
            lt[l] = t;
            base += ((t.H + TH - 1) / TH) * t.ntx;
        }
        *total = base;
    }
    __syncthreads();
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ inline uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// within each row of 16 lanes (lanes shifted in from outside the row read 0),
// then the last lane of row 0 is added to row 1 and 3 (row broadcast 15) and
// the last lane of row 1 to rows 2 and 3 (row broadcast 31).
__device__ inline uint32_t wave_inclusive_scan(uint32_t x) {
    x += dpp_u32<0x111, 0xF, true>(x);   // row_shr:1
    x += dpp_u32<0x112, 0xF, true>(x);   // row_shr:2
    x += dpp_u32<0x114, 0xF, true>(x);   // row_shr:4
    x += dpp_u32<0x118, 0xF, true>(x);   // row_shr:8
    x += dpp_u32<0x142, 0xA, false>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_u32<0x143, 0xC, false>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Exclusive scan of a[0, n) into o[0, n) by the whole block; returns the total
// to every thread. Each thread takes a contiguous segment, the segment sums
// are scanned per wave with DPP and the wave totals combined through LDS.
// a and o may alias; scratch holds kWavesPerBlock words.
__device__ inline uint32_t block_exclusive_scan(const uint32_t* a, uint32_t* o, int n,
                                                uint32_t* scratch) {
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int per = (n + kBlock - 1) / kBlock;
    const int lo = min(tid * per, n), hi = min(lo + per, n);
    uint32_t s = 0;
    for (int i = lo; i < hi; ++i) s += a[i];
    const uint32_t incl = wave_inclusive_scan(s);
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        const uint32_t t = scratch[w];
        base += w < wave ? t : 0u;
        total += t;
    }
    uint32_t run = base + incl - s;
    for (int i = lo; i < hi; ++i) {
        const uint32_t v = a[i];
        o[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

// The distinct tiles (local indices in the (b, m)) that a point's
// inside-the-level corners fall in, without loops or branches: tile[c] is the
// tile of corner c (0: (y0,x0), 1: (y0,x0+1), 2: (y0+1,x0), 3: (y0+1,x0+1))
// and emit[c] says whether corner c is inside the level and is the first
// corner of its tile.
// (u, v) normalized, or with kPixel already the pixel coordinates (x, y).
template <int TW, int TH, bool kPixel>
__device__ inline void point_tiles(float u, float v, const LevelTiles& lt, int* tile, bool* emit) {
    const float Hf = (float)lt.H, Wf = (float)lt.W;
    const float x = kPixel ? u : fmaf(u, Wf, -0.5f);
    const float y = kPixel ? v : fmaf(v, Hf, -0.5f);
    const float x0f = floorf(x), y0f = floorf(y);
    const bool vx0 = (x0f >= 0.0f) && (x0f < Wf);
    const bool vx1 = (x0f >= -1.0f) && (x0f < Wf - 1.0f);
    const bool vy0 = (y0f >= 0.0f) && (y0f < Hf);
    const bool vy1 = (y0f >= -1.0f) && (y0f < Hf - 1.0f);
    const int x0 = (int)fminf(fmaxf(x0f, -1.0f), Wf);
    const int y0 = (int)fminf(fmaxf(y0f, -1.0f), Hf);
    // tile coordinates of the two columns and rows (only used where valid,
    // i.e. where the pixel coordinate is >= 0)
    const int tx0 = (int)((uint32_t)max(x0, 0) / (uint32_t)TW);
    const int tx1 = (int)((uint32_t)(x0 + 1) / (uint32_t)TW);
    const int ty0 = max(y0, 0) / TH, ty1 = (y0 + 1) / TH;
    const bool v00 = vx0 && vy0, v01 = vx1 && vy0, v10 = vx0 && vy1, v11 = vx1 && vy1;
    const bool same_x = tx0 == tx1, same_y = ty0 == ty1;
    emit[0] = v00;
    emit[1] = v01 && !(v00 && same_x);
    emit[2] = v10 && !(v00 && same_y);
    emit[3] = v11 && !(v01 && same_y) && !(v10 && same_x) && !(v00 && same_x && same_y);
    const int r0 = lt.tile_base + ty0 * lt.ntx, r1 = lt.tile_base + ty1 * lt.ntx;
    tile[0] = r0 + tx0;
    tile[1] = r0 + tx1;
    tile[2] = r1 + tx0;
    tile[3] = r1 + tx1;
}

// Walks the points of one bin block (queries [q_begin, ...) of one (b, m)) with
// a stride of kBlock, keeping the query offset, point slot j, level l, tuple
// and global point index up to date without a division per point.
struct PointWalk {
    int i, qo, j, l, dq, dj, LK, K;
    float invK;
    size_t t, pt;
    size_t tuple0;  // (b*Nq + q_begin)*M + m
    size_t pt0;     // the walk's first point (valid whenever the walk is not empty)
    int M;
    __device__ PointWalk(const Params& p, int tid, int q_begin, int b, int m)
        : i(tid), LK(p.LK > 0 ? p.LK : 1), K(p.K > 0 ? p.K : 1), M(p.M) {
        invK = 1.0f / (float)K;
        qo = i / LK;
        j = i - qo * LK;
        dq = kBlock / LK;
        dj = kBlock - dq * LK;
        tuple0 = ((size_t)b * p.Nq + q_begin) * p.M + m;
        pt0 = tuple0 * LK;
        update();
    }
    __device__ void update() {
        // j / K through the reciprocal, corrected by one step either way
        l = (int)((float)j * invK);
        l -= (l * K > j);
        l += ((l + 1) * K <= j);
        t = tuple0 + (size_t)qo * M;
        pt = t * LK + j;
    }
    __device__ void next() {
        i += kBlock;
        qo += dq;
        j += dj;
        if (j >= LK) {
            j -= LK;
            ++qo;
        }
        update();
    }
};

// kCached: the block has at most kBinUnroll points per thread, loaded once and
// kept in registers for both passes (otherwise each pass loads them).
// All but the DCNv3 front-end: the entries bound for the first kBinStage
// slots of the block's slab (of the current tile range) are written to LDS
// first and copied out in order, whole lines at a time; scattered 16-byte
// stores to the slab touch one cache line per lane. Sized so that the LDS
// still holds as many blocks per CU as the registers allow (4 cached, 5 not).
// (DCNv3 measured slower with it: 141 -> 155 us for its grad_input stage.)
template <int FE, bool kCached>
constexpr int bin_stage() {
    return FE != kFeDcn ? (kCached ? 2000 : 1488) : 0;
}

template <int D, int FE, int TH, bool kCached>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(kCached && bin_stage<FE, kCached>() > 0 ? 4 : 1)))
void msda_bin_kernel(Params p) {
    using TS = TileShape<D, TH>;
    constexpr int kStage = bin_stage<FE, kCached>();
    __shared__ LevelTiles lt[MSDA_MAX_LEVELS];
    __shared__ int s_tiles;
    __shared__ uint32_t cnt[kBinRange];
    __shared__ uint32_t off[kBinRange];
    __shared__ uint32_t scratch[kWavesPerBlock];
    __shared__ float4 staged[kStage > 0 ? kStage : 1];
    setup_tiles<TS::TW, TH>(p, lt, &s_tiles);
    // tables inconsistent with Nv could exceed the row: drop those tiles
    // rather than write past the workspace
    const int T = block_uniform(min(s_tiles, p.t_stride - 1));
    const int tid = threadIdx.x;
    const int bml = blockIdx.x / p.nW, w = blockIdx.x - bml * p.nW;   // plane of the pass
    const int bm = p.bm0 + bml;
    const int b = bm / p.M, m = bm - b * p.M;
    const int q_begin = min(w * p.Qc, p.Nq), q_end = min(q_begin + p.Qc, p.Nq);
    const int npts = (q_end - q_begin) * p.LK;
    // this block's column of the (tile, bin block) table of its (b, m)
    uint32_t* row = p.table + (size_t)bml * p.t_stride * p.nW + w;
    float4* slab = p.slab + (size_t)blockIdx.x * p.slab_per_block;
    if (blockIdx.x == 0 && tid < 8) p.counters[tid * kCounterStride] = 0;   // for the tile kernel that follows
    // location (and weight) of the walk's current point, or of its first point
    // for lanes past the end, so that every load is unconditional
    // (normalized, or for the DCNv3 front-end in pixels)
    auto point_of = [&](const PointWalk& it, bool ok, float2& uv, float& a, bool want_a) {
        if constexpr (FE != kFeCore) {
            const int t = ok ? (int)it.t : (int)it.tuple0;
            const int j = ok ? it.j : 0;
            const int l = ok ? it.l : 0;
            const int q = ok ? q_begin + it.qo : q_begin;
            float2 st = make_float2(0.f, 0.f);
            if constexpr (FE == kFeFused) st = want_a ? p.smax[t] : st;
            finish_point<FE>(load_point_q<FE>(p, t, j, l, q),
                             make_int4(lt[l].H, lt[l].W, lt[l].start, 0), st.x, st.y, uv, a);
        } else {
            const size_t pt = ok ? it.pt : it.pt0;
            uv = *reinterpret_cast<const float2*>(p.loc + 2 * pt);
            a = want_a ? p.attn[pt] : 0.0f;
        }
    };
    uint32_t base = 0;
    if constexpr (kCached) {
        // the pixel coordinates (x, y) of a point, its level, tuple and weight
        float px[kBinUnroll], py[kBinUnroll], pa[kBinUnroll];
        int lvl[kBinUnroll];
        bool ok[kBinUnroll];
        uint32_t tup[kBinUnroll];
        {
            PointWalk it(p, tid, q_begin, b, m);
            float2 uv[kBinUnroll];
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                ok[u] = it.i < npts;
                lvl[u] = it.l;
                tup[u] = (uint32_t)it.t;
                point_of(it, ok[u], uv[u], pa[u], true);
                it.next();
            }
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                const LevelTiles& L_ = lt[lvl[u]];
                px[u] = FE == kFeDcn ? uv[u].x : fmaf(uv[u].x, (float)L_.W, -0.5f);
                py[u] = FE == kFeDcn ? uv[u].y : fmaf(uv[u].y, (float)L_.H, -0.5f);
            }
        }
        for (int r0 = 0; r0 < T; r0 += kBinRange) {
            const int rn = min(kBinRange, T - r0);
            for (int i = tid; i < rn; i += kBlock) cnt[i] = 0;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                int tile[4];
                bool emit[4];
                point_tiles<TS::TW, TH, true>(px[u], py[u], lt[lvl[u]], tile, emit);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (ok[u] && emit[c] && tile[c] >= r0 && tile[c] < r0 + rn)
                        atomicAdd(&cnt[tile[c] - r0], 1u);
                }
            }
            __syncthreads();
            const uint32_t total = block_exclusive_scan(cnt, off, rn, scratch);
            for (int i = tid; i < rn; i += kBlock) row[(size_t)(r0 + i) * p.nW] = base + off[i];
            __syncthreads();
            for (int i = tid; i < rn; i += kBlock) cnt[i] = 0;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                int tile[4];
                bool emit[4];
                point_tiles<TS::TW, TH, true>(px[u], py[u], lt[lvl[u]], tile, emit);
                const float4 rec = make_float4(as_float(tup[u]), px[u], py[u], pa[u]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (ok[u] && emit[c] && tile[c] >= r0 && tile[c] < r0 + rn) {
                        const uint32_t pos = off[tile[c] - r0] + atomicAdd(&cnt[tile[c] - r0], 1u);
                        if (pos < (uint32_t)kStage)
                            staged[pos] = rec;
                        else
                            slab[base + pos] = rec;
                    }
                }
            }
            if constexpr (kStage > 0) {
                __syncthreads();
                for (uint32_t i = tid; i < min(total, (uint32_t)kStage); i += kBlock) {
                    if (p.slab_streaming)
                        store_streaming(slab + base + i, staged[i]);
                    else
                        slab[base + i] = staged[i];
                }
            }
            base += total;
            __syncthreads();
        }
        if (tid == 0) row[(size_t)T * p.nW] = base;   // end of the last tile's entries
        return;
    }
    // a point index that is always valid (npts > 0 whenever a loop body runs)
    // stands in for the lanes past the end, so that every load is unconditional
    for (int r0 = 0; r0 < T; r0 += kBinRange) {
        const int rn = min(kBinRange, T - r0);
        for (int i = tid; i < rn; i += kBlock) cnt[i] = 0;
        __syncthreads();
        for (PointWalk it(p, tid, q_begin, b, m); it.i < npts;) {
            float2 uv[kBinUnroll];
            int lvl[kBinUnroll];
            bool ok[kBinUnroll];
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                ok[u] = it.i < npts;
                lvl[u] = it.l;
                float a_unused;
                point_of(it, ok[u], uv[u], a_unused, false);
                it.next();
            }
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                int tile[4];
                bool emit[4];
                point_tiles<TS::TW, TH, FE == kFeDcn>(uv[u].x, uv[u].y, lt[lvl[u]], tile, emit);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (ok[u] && emit[c] && tile[c] >= r0 && tile[c] < r0 + rn)
                        atomicAdd(&cnt[tile[c] - r0], 1u);
                }
            }
        }
        __syncthreads();
        const uint32_t total = block_exclusive_scan(cnt, off, rn, scratch);
        for (int i = tid; i < rn; i += kBlock) row[(size_t)(r0 + i) * p.nW] = base + off[i];
        __syncthreads();
        for (int i = tid; i < rn; i += kBlock) cnt[i] = 0;
        __syncthreads();
        for (PointWalk it(p, tid, q_begin, b, m); it.i < npts;) {
            float2 uv[kBinUnroll];
            float a[kBinUnroll];
            int lvl[kBinUnroll];
            bool ok[kBinUnroll];
            uint32_t tup[kBinUnroll];
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                ok[u] = it.i < npts;
                lvl[u] = it.l;
                tup[u] = (uint32_t)it.t;
                point_of(it, ok[u], uv[u], a[u], true);
                it.next();
            }
#pragma unroll
            for (int u = 0; u < kBinUnroll; ++u) {
                int tile[4];
                bool emit[4];
                const LevelTiles& L_ = lt[lvl[u]];
                point_tiles<TS::TW, TH, FE == kFeDcn>(uv[u].x, uv[u].y, L_, tile, emit);
                // the entry carries all the tile kernel needs: the tuple (its
                // upstream-gradient row), the fp32 pixel coordinates (cell and
                // fractions follow from them exactly as here) and the weight
                const float px = FE == kFeDcn ? uv[u].x : fmaf(uv[u].x, (float)L_.W, -0.5f);
                const float py = FE == kFeDcn ? uv[u].y : fmaf(uv[u].y, (float)L_.H, -0.5f);
                const float4 rec = make_float4(as_float(tup[u]), px, py, a[u]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (ok[u] && emit[c] && tile[c] >= r0 && tile[c] < r0 + rn) {
                        const uint32_t pos = off[tile[c] - r0] + atomicAdd(&cnt[tile[c] - r0], 1u);
                        if (pos < (uint32_t)kStage)
                            staged[pos] = rec;
                        else
                            slab[base + pos] = rec;
                    }
                }
            }
        }
        if constexpr (kStage > 0) {
            __syncthreads();
            for (uint32_t i = tid; i < min(total, (uint32_t)kStage); i += kBlock) {
                if (p.slab_streaming)
                    store_streaming(slab + base + i, staged[i]);
                else
                    slab[base + i] = staged[i];
            }
        }
        base += total;
        __syncthreads();
    }
    if (tid == 0) row[(size_t)T * p.nW] = base;   // end of the last tile's entries
}

// One work item = one tile of one (b, m). Work items are fetched dynamically
// from a counter per XCD group (blocks i = x mod 8 run on XCD x and serve the
// (b, m) = x mod 8, so an XCD's L2 sees only its own (b, m)), coarse levels
// first: those tiles have the most points per pixel and the longest lists, and
// start first. A block takes the tile's entries kChunk at a time: loads them,
// counting-sorts them by cell into LDS records that already hold the four
// corner weights, then sweeps the cells column by column. (Tall tiles: at
// most 128 VGPRs, so that 4 blocks fit per CU.)
template <int D, bool kBf16Out, int TH>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(TH == kTileHTall ? 4 : 1)))
void msda_tile_kernel(Params p) {
    using TS = TileShape<D, TH>;
    constexpr int TW = TS::TW, NG = TS::NG, G = TS::G, kCells = TS::kCells;
    // the column exchange reuses the record buffer, kXch pixel rows at a
    // time; the zero record sits after the chunk's records
    constexpr int kXch = kChunk / kBlock < TH ? kChunk / kBlock : TH;
    static_assert(TH % kXch == 0, "exchange rows");
    constexpr int kZero = kChunk;
    // Tall tiles (sparse points) order the cells column by column, so that a
    // lane group's entries form one range and all its loads go out together
    // (a cell-row-by-row sweep waits for one load round trip per non-empty
    // cell row of the wave's columns); each record then carries its cell row
    // in the low bits of the row offset (a multiple of 4 D >= 32).
    constexpr bool kColMajor = TH == kTileHTall;
    static_assert(!kColMajor || (TH < 16 && D * sizeof(float) >= 16), "cell row in the offset's low bits");
    constexpr int kPer = kChunk / kBlock;   // entries per thread per chunk
    static_assert(kPer * kBlock == kChunk, "chunk size");
    __shared__ LevelTiles lt[MSDA_MAX_LEVELS];
    __shared__ int s_tiles, s_item;
    __shared__ uint32_t wcnt[kMaxSlabs], wstart[kMaxSlabs], woff[kMaxSlabs];
    // a chunk's entries in cell order: the four corner weights (top-left,
    // top-right, bottom-left, bottom-right) and the byte offset of the
    // upstream-gradient row
    // (slot kZero: a zero record for the sweep's slots past a range's end)
    __shared__ float4 wrec[kZero + 1];
    __shared__ uint32_t grec[kZero + 1];
    __shared__ uint32_t cstart[kCells + 1];
    __shared__ uint32_t ccount[kCells + 1];
    __shared__ uint32_t scratch[kWavesPerBlock];
    if (threadIdx.x == 0) {
        wrec[kZero] = make_float4(0.f, 0.f, 0.f, 0.f);
        grec[kZero] = kOutside;   // out of the buffer's range: loads zeros
    }
    setup_tiles<TW, TH>(p, lt, &s_tiles);
    const int T = block_uniform(min(s_tiles, p.t_stride - 1));
    const int tid = threadIdx.x;
    const int BM = p.bm_count;   // the planes of this pass
    const int col = tid / G, r = tid % G;
    // upstream-gradient rows through a buffer descriptor: 32-bit offsets
    const __amdgpu_buffer_rsrc_t grsrc =
        make_rsrc(p.grad_out, (uint32_t)((size_t)p.T * D * sizeof(float)));
    const __amdgpu_buffer_rsrc_t gvrsrc = make_rsrc(p.grad_value, p.grad_value_bytes);

    const int xcd = blockIdx.x % 8;
    const int nbm_x = BM >= 8 ? (BM - xcd + 7) / 8 : 0;
    const int items = BM >= 8 ? nbm_x * T : (BM * T - xcd + 7) / 8;
    uint32_t* const counter = p.counters + xcd * kCounterStride;
    for (;;) {
        if (tid == 0) s_item = (int)atomicAdd(counter, 1u);
        __syncthreads();
        const int k = block_uniform(s_item);
        if (k >= items) break;
        int bm, tl;
        if (BM >= 8) {
            bm = xcd + 8 * (k % nbm_x);
            tl = T - 1 - k / nbm_x;
        } else {
            const int i = xcd + 8 * k;
            bm = i % BM;
            tl = T - 1 - i / BM;
        }
        int l = 0;
        while (l + 1 < p.L && lt[l + 1].tile_base <= tl) ++l;
        const LevelTiles L_ = lt[l];
        const int ty = (tl - L_.tile_base) / L_.ntx, tx = (tl - L_.tile_base) - ty * L_.ntx;
        const int y_base = ty * TH, x_base = tx * TW;
        const int b = (p.bm0 + bm) / p.M, m = (p.bm0 + bm) - b * p.M;

        // this tile's entries in every slab of (b, m): rows tl and tl + 1 of
        // the table hold where they start and end
        const uint32_t* trow = p.table + ((size_t)bm * p.t_stride + tl) * p.nW;
        for (int w = tid; w < p.nW; w += kBlock) {
            const uint32_t lo = trow[w];
            wcnt[w] = trow[p.nW + w] - lo;
            woff[w] = lo;
        }
        __syncthreads();
        const uint32_t E = (uint32_t)block_uniform((int)block_exclusive_scan(wcnt, wstart, p.nW, scratch));

        float4 own[TH], prev[TH];
#pragma unroll
        for (int y = 0; y < TH; ++y) {
            own[y] = make_float4(0.f, 0.f, 0.f, 0.f);
            prev[y] = own[y];
        }

        for (uint32_t c0 = 0; c0 < E; c0 += kChunk) {
            const int n = (int)min((uint32_t)kChunk, E - c0);
            for (int i = tid; i <= kCells; i += kBlock) ccount[i] = 0;
            __syncthreads();
            // every thread takes entries tid + j * kBlock of the chunk, all
            // kPer loads in flight (indices past the end re-read the last entry)
            float4 ent[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const uint32_t ge = c0 + min(tid + j * kBlock, n - 1);
                int lo = 0;   // last slab whose start <= ge (nW <= kMaxSlabs)
#pragma unroll
                for (int step = kMaxSlabs / 2; step > 0; step >>= 1) {
                    const int probe = min(lo + step, p.nW - 1);
                    lo = wstart[probe] <= ge ? probe : lo;
                }
                ent[j] = load_streaming(p.slab + ((size_t)bm * p.nW + lo) * p.slab_per_block +
                                        woff[lo] + (ge - wstart[lo]));
            }
            // cell of each entry; histogram
            int cell[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                // an entry has a corner in this tile, so its cell is within
                // one pixel of it; clamp anyway to stay in bounds
                const int cy = min(max((int)floorf(ent[j].z) - y_base, -1), TH - 1);
                const int cx = min(max((int)floorf(ent[j].y) - x_base, -1), TW - 1);
                cell[j] = kColMajor ? (cx + 1) * (TH + 1) + (cy + 1) : (cy + 1) * NG + (cx + 1);
                if (tid + j * kBlock < n) atomicAdd(&ccount[cell[j]], 1u);
            }
            __syncthreads();
            block_exclusive_scan(ccount, cstart, kCells + 1, scratch);
            for (int i = tid; i <= kCells; i += kBlock) ccount[i] = 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (tid + j * kBlock < n) {
                    const uint32_t slot = cstart[cell[j]] + atomicAdd(&ccount[cell[j]], 1u);
                    const float x = ent[j].y, y = ent[j].z, a = ent[j].w;
                    const float fx = x - floorf(x), fy = y - floorf(y);
                    const float at = a * (1.0f - fy), ab = a * fy;
                    wrec[slot] = make_float4(at * (1.0f - fx), at * fx, ab * (1.0f - fx), ab * fx);
                    grec[slot] = as_uint(ent[j].x) * (uint32_t)(D * sizeof(float)) +
                                 (kColMajor ? (uint32_t)(cell[j] % (TH + 1)) : 0u);
                }
            }
            __syncthreads();
            // cell-column sweep: lane group col takes the cells of cell column
            // col - 1 and adds each entry's right corners to pixel column col
            // (own) and its left corners to pixel column col - 1 (prev), one
            // upstream-gradient row per entry. kUnroll entries are in flight
            // at once; slots past the end of the group's range read the zero
            // record.
            const uint32_t lane_off = (uint32_t)r * 16u;
            if constexpr (kColMajor) {
                // the column's cells in one range; a cell in cell row cr has
                // its top corners on pixel row cr - 1 and its bottom corners
                // on pixel row cr, picked per entry (a product is added only
                // to its own rows, so a non-finite gradient stays there)
                const uint32_t s0 = cstart[col * (TH + 1)], e = cstart[(col + 1) * (TH + 1)];
                for (uint32_t k = s0; k < e; k += kUnrollTall) {
                    const uint32_t rem = e - k;
                    float4 gv[kUnrollTall], wv[kUnrollTall];
                    int crow[kUnrollTall];
#pragma unroll
                    for (int u = 0; u < kUnrollTall; ++u) {
                        const uint32_t si = (uint32_t)u < rem ? k + u : (uint32_t)kZero;
                        wv[u] = wrec[si];
                        const uint32_t gr = grec[si];
                        crow[u] = (int)(gr & 15u);
                        const u32x4 graw = __builtin_amdgcn_raw_buffer_load_b128(
                            grsrc, (gr & ~15u) + lane_off, 0, 0);
                        gv[u] = make_float4(as_float(graw[0]), as_float(graw[1]),
                                            as_float(graw[2]), as_float(graw[3]));
                    }
#pragma unroll
                    for (int u = 0; u < kUnrollTall; ++u) {
#pragma unroll
                        for (int y = 0; y < TH; ++y) {
                            const bool top = y == crow[u] - 1, bot = y == crow[u];
                            const float wl = top ? wv[u].x : wv[u].z;
                            const float wr = top ? wv[u].y : wv[u].w;
                            if (top || bot) {
                                prev[y].x = fmaf(wl, gv[u].x, prev[y].x);
                                prev[y].y = fmaf(wl, gv[u].y, prev[y].y);
                                prev[y].z = fmaf(wl, gv[u].z, prev[y].z);
                                prev[y].w = fmaf(wl, gv[u].w, prev[y].w);
                                own[y].x = fmaf(wr, gv[u].x, own[y].x);
                                own[y].y = fmaf(wr, gv[u].y, own[y].y);
                                own[y].z = fmaf(wr, gv[u].z, own[y].z);
                                own[y].w = fmaf(wr, gv[u].w, own[y].w);
                            }
                        }
                    }
                }
            } else {
#pragma unroll
                for (int cr = 0; cr <= TH; ++cr) {   // cell row cy = cr - 1
                    const int lc = cr * NG + col;
                    const uint32_t s0 = cstart[lc], e = cstart[lc + 1];
                    for (uint32_t k = s0; k < e; k += kUnroll) {
                        const uint32_t rem = e - k;
                        float4 gv[kUnroll], wv[kUnroll];
#pragma unroll
                        for (int u = 0; u < kUnroll; ++u) {
                            const uint32_t si = (uint32_t)u < rem ? k + u : (uint32_t)kZero;
                            wv[u] = wrec[si];
                            const u32x4 graw = __builtin_amdgcn_raw_buffer_load_b128(
                                grsrc, grec[si] + lane_off, 0, 0);
                            gv[u] = make_float4(as_float(graw[0]), as_float(graw[1]),
                                                as_float(graw[2]), as_float(graw[3]));
                        }
#pragma unroll
                        for (int u = 0; u < kUnroll; ++u) {
                            {
                                // a cell in cell row cr has its top corners on pixel
                                // row cr - 1 and its bottom corners on pixel row cr
                                if (cr >= 1) {
                                    prev[cr - 1].x = fmaf(wv[u].x, gv[u].x, prev[cr - 1].x);
                                    prev[cr - 1].y = fmaf(wv[u].x, gv[u].y, prev[cr - 1].y);
                                    prev[cr - 1].z = fmaf(wv[u].x, gv[u].z, prev[cr - 1].z);
                                    prev[cr - 1].w = fmaf(wv[u].x, gv[u].w, prev[cr - 1].w);
                                    own[cr - 1].x = fmaf(wv[u].y, gv[u].x, own[cr - 1].x);
                                    own[cr - 1].y = fmaf(wv[u].y, gv[u].y, own[cr - 1].y);
                                    own[cr - 1].z = fmaf(wv[u].y, gv[u].z, own[cr - 1].z);
                                    own[cr - 1].w = fmaf(wv[u].y, gv[u].w, own[cr - 1].w);
                                }
                                if (cr < TH) {
                                    prev[cr].x = fmaf(wv[u].z, gv[u].x, prev[cr].x);
                                    prev[cr].y = fmaf(wv[u].z, gv[u].y, prev[cr].y);
                                    prev[cr].z = fmaf(wv[u].z, gv[u].z, prev[cr].z);
                                    prev[cr].w = fmaf(wv[u].z, gv[u].w, prev[cr].w);
                                    own[cr].x = fmaf(wv[u].w, gv[u].x, own[cr].x);
                                    own[cr].y = fmaf(wv[u].w, gv[u].y, own[cr].y);
                                    own[cr].z = fmaf(wv[u].w, gv[u].z, own[cr].z);
                                    own[cr].w = fmaf(wv[u].w, gv[u].w, own[cr].w);
                                }
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
        // pixel column col = own (cell column col - 1) + the prev sums of lane
        // group col + 1 (cell column col), passed through the record buffer,
        // which no thread reads any more
        float4* xch = wrec;
#pragma unroll
        for (int h = 0; h < TH; h += kXch) {
            if (h > 0) __syncthreads();   // the previous rows have been read
#pragma unroll
            for (int yy = 0; yy < kXch; ++yy) xch[yy * kBlock + tid] = prev[h + yy];
            __syncthreads();
            if (col < TW) {
#pragma unroll
                for (int yy = 0; yy < kXch; ++yy) {
                    const float4 nb = xch[yy * kBlock + tid + G];
                    own[h + yy].x += nb.x;
                    own[h + yy].y += nb.y;
                    own[h + yy].z += nb.z;
                    own[h + yy].w += nb.w;
                }
            }
        }
        // every pixel of the tile that is inside the level, written once,
        // through a buffer descriptor: level tables inconsistent with Nv (the
        // caller's contract, not checked on the device) cannot write past
        // grad_value -- such a store lands beyond the record count and is
        // dropped. Non-temporal: no later tile reads it, and the L2 is
        // better spent on the upstream-gradient rows the tiles share.
        const int x = x_base + col;
        if (col < TW && x < L_.W) {
#pragma unroll
            for (int yy = 0; yy < TH; ++yy) {
                const int y = y_base + yy;
                if (y < L_.H) {
                    const uint64_t rowi = (uint64_t)b * p.Nv + L_.start + (uint64_t)y * L_.W + x;
                    const uint64_t byte = ((rowi * p.M + m) * D + r * 4) * (kBf16Out ? 2 : 4);
                    const uint32_t voff = byte < p.grad_value_bytes ? (uint32_t)byte : kOutside;
                    if constexpr (kBf16Out) {
                        // rounded once, from the fp32 sum
                        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                        const u32x2 v = {float_to_bf16_bits(own[yy].x) | (float_to_bf16_bits(own[yy].y) << 16),
                                         float_to_bf16_bits(own[yy].z) | (float_to_bf16_bits(own[yy].w) << 16)};
                        __builtin_amdgcn_raw_buffer_store_b64(v, gvrsrc, voff, 0, kBufferNonTemporal);
                    } else {
                        const u32x4 v = {as_uint(own[yy].x), as_uint(own[yy].y), as_uint(own[yy].z),
                                         as_uint(own[yy].w)};
                        __builtin_amdgcn_raw_buffer_store_b128(v, gvrsrc, voff, 0, kBufferNonTemporal);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ fused front-end
// Softmax statistics of every tuple's L*K logits: (max, 1 / sum exp(z - max)),
// one thread per tuple.
__global__ __launch_bounds__(kBlock) void msda_softmax_stats_kernel(Params p) {
    // a quad of lanes per tuple: with L*K a multiple of 4 (and 16-byte aligned
    // logits) each lane reads whole float4s, so the quads of a wave read one
    // contiguous run of logits. Grid-stride over tuples; a quad's lanes always
    // share their tuple, so all four take part in the quad reductions.
    const int i = threadIdx.x & 3;
    const bool vec = (p.LK & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
    const int n4 = p.LK >> 2;
    const int64_t stride = (int64_t)gridDim.x * (kBlock / 4);
    for (int64_t t = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 2; t < p.T; t += stride) {
        const float* z = p.logits + t * p.LK;
        const float4* z4 = reinterpret_cast<const float4*>(z);
        float mx = -INFINITY;
        if (vec) {
            for (int f = i; f < n4; f += 4) {
                const float4 v = z4[f];
                mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            }
        } else {
            for (int j = i; j < p.LK; j += 4) mx = fmaxf(mx, z[j]);
        }
        mx = fmaxf(mx, dpp<0xB1>(mx));   // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp<0x4E>(mx));   // quad_perm [2,3,0,1]
        float se = 0.0f;
        if (vec) {
            for (int f = i; f < n4; f += 4) {
                const float4 v = z4[f];
                se += (expf(v.x - mx) + expf(v.y - mx)) + (expf(v.z - mx) + expf(v.w - mx));
            }
        } else {
            for (int j = i; j < p.LK; j += 4) se += expf(z[j] - mx);
        }
        se = group_sum<4>(se);
        if (i == 0) p.smax[t] = make_float2(mx, 1.0f / se);
    }
}

// Gradient of a reference point: every head's and point's location on its
// level moves with it, so dL/dref[b,q,l] = sum over m, k of dL/dloc, where
// dL/dloc = dL/doff * (W, H). One thread per (b, q, l).
__global__ __launch_bounds__(kBlock) void msda_ref_grad_kernel(Params p, float* grad_ref) {
    const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;   // (b*Nq + q)*L + l
    if (i >= (size_t)p.B * p.Nq * p.L) return;
    const size_t bq = i / p.L;
    const int l = (int)(i - bq * p.L);
    const float Hf = (float)p.shapes[2 * l], Wf = (float)p.shapes[2 * l + 1];
    float gx = 0.0f, gy = 0.0f;
    for (int m = 0; m < p.M; ++m) {
        const float2* g = reinterpret_cast<const float2*>(p.grad_off) +
                          ((bq * p.M + m) * p.L + l) * p.K;
        for (int k = 0; k < p.K; ++k) {
            const float2 v = g[k];
            gx += v.x;
            gy += v.y;
        }
    }
    reinterpret_cast<float2*>(grad_ref)[i] = make_float2(gx * Wf, gy * Hf);
}

// ------------------------------------------------------------------ host side
constexpr int64_t k2GiB = int64_t(1) << 31;
constexpr size_t kWorkspaceAlign = 256;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b <= limit for non-negative a, b, without overflow
bool mul_le(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

// Host checks shared by both entry points. Every offset the kernels form is
// 32-bit: the value, grad_value and output tensors must stay below 2 GiB, the
// point count below 2^31.
msda_status_t check_dims(const msda_dims_t* d, msda_dtype_t dt, bool backward) {
    if (!d) return MSDA_ERROR_INVALID_VALUE;
    if (d->B < 0 || d->Nq < 0 || d->K < 0 || d->M < 1 || d->Nv < 1 || d->L < 1 || d->D < 1)
        return MSDA_ERROR_INVALID_VALUE;
    if (dt != MSDA_DTYPE_F32 && dt != MSDA_DTYPE_BF16 && dt != MSDA_DTYPE_F16)
        return MSDA_ERROR_INVALID_VALUE;
    if (d->L > MSDA_MAX_LEVELS) return MSDA_ERROR_NOT_SUPPORTED;
    if (d->D != 8 && d->D != 16 && d->D != 32 && d->D != 64) return MSDA_ERROR_NOT_SUPPORTED;
    const int64_t lim = k2GiB - 1;
    const int64_t elem = (backward || dt == MSDA_DTYPE_F32) ? 4 : 2;  // widest value-shaped buffer
    if (!mul_le(d->Nv, d->M, lim) || !mul_le(d->Nv * d->M, d->D * elem, lim) ||
        !mul_le(d->B, d->Nv * d->M * d->D * elem, lim))
        return MSDA_ERROR_NOT_SUPPORTED;
    // output / grad_output bytes
    if (!mul_le(d->Nq, d->M, lim) || !mul_le(d->Nq * d->M, d->D * 4, lim) ||
        !mul_le(d->B, d->Nq * d->M * d->D * 4, lim))
        return MSDA_ERROR_NOT_SUPPORTED;
    // points (x2 for the location pairs)
    if (!mul_le(d->L, d->K, lim / 2) || !mul_le(d->B * d->Nq * d->M, d->L * d->K * 2, lim))
        return MSDA_ERROR_NOT_SUPPORTED;
    return MSDA_SUCCESS;
}

// Workspace of the grad_value path (bin + tile kernels): 8 work counters of
// the tile kernel (kCounterStride words apart), then, for each (b, m) plane of
// a pass, nW bin blocks each owning Qc queries, a table of nW slab offsets per
// tile boundary and a slab of 16-byte entries per bin block (at most 4 per
// point: one per tile its inside corners fall in). The tile count of one
// (b, m) is bounded from Nv and L alone: a level of H x W pixels has
// ceil(H/4) ceil(W/TW) tiles (TW >= 15), which is at most H/4 + 3/4 when
// W <= TW and below (H+3) W / (2 TW) <= 2 H W / 15 otherwise, so
// sum_l <= Nv/4 + L, and the table has Nv/4 + L + 1 rows per (b, m).
//
// The planes are binned and swept in passes of bm_per_pass planes that share
// the workspace: the bytes per plane are fixed by the sizes, so a workspace
// of any size from one plane's up to all planes' (one pass, the fastest) is
// used in as few passes as it allows. Passes of a multiple of 8 planes keep
// the tile kernel's 8 XCD groups busy alike.
struct BwdPlan {
    int64_t nW = 0, Qc = 0, t_stride = 0, slab_per_block = 0;
    int64_t bm_per_pass = 0, passes = 0;
    int tall = 0;   // tiles of kTileHTall rows (1) or kTileH rows (0)
    int cached = 0; // bin blocks of at most kBinUnroll points per thread (1)
    size_t counters_off = 0, table_off = 0, slab_off = 0, bytes = 0;
    size_t min_bytes = 0;   // the workspace of one plane per pass
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr size_t kCountersBytes = 8 * kCounterStride * sizeof(uint32_t);

// The plan for a workspace of at most `budget` bytes (the fewest passes that
// fit; bytes = 0 when not even one plane fits).
BwdPlan plan_backward(const msda_dims_t* d, size_t budget = SIZE_MAX) {
    BwdPlan pl;
    const int64_t BM = d->B * d->M;
    if (BM == 0) return pl;
    // about 4096 bin blocks in total, at most kBinSlabs per (b, m) and at
    // least kMinQueries queries per block (fewer, fuller slabs when there are
    // few queries: every tile reads one table entry per slab)
    int64_t nW = (4096 + BM - 1) / BM;
    nW = nW < 1 ? 1 : (nW > kBinSlabs ? kBinSlabs : nW);
    const int64_t nW_q = (d->Nq + kMinQueries - 1) / kMinQueries;
    if (nW > nW_q) nW = nW_q < 1 ? 1 : nW_q;
    // more, smaller bin blocks where that lets every block keep its points
    // in registers (one load per point instead of one per pass), as long as
    // the (tile, block) table -- nW rows per tile -- grows at most threefold
    const int64_t LK = d->L * d->K;
    const int64_t q_fit = LK > 0 ? (int64_t)(kBinUnroll * kBlock) / LK : 0;
    if (q_fit >= 1 && d->Nq > 0) {
        const int64_t nW_fit = (d->Nq + q_fit - 1) / q_fit;
        if (nW_fit <= kMaxSlabs && nW_fit <= 3 * nW) {
            if (nW_fit > nW) nW = nW_fit;
            pl.cached = 1;
        }
    }
    const int64_t Qc = d->Nq > 0 ? (d->Nq + nW - 1) / nW : 0;
    pl.nW = Qc > 0 ? (d->Nq + Qc - 1) / Qc : 1;
    pl.Qc = Qc;
    pl.t_stride = (d->Nv + 3) / 4 + d->L + 1;
    static_assert(kTileH >= 4 && kTileHTall >= 4, "the tile-count bound above assumes tiles of 4 rows or more");
    // tall tiles where a (b, m) has fewer points than pixels
    pl.tall = d->Nq * d->L * d->K < d->Nv ? 1 : 0;
    pl.slab_per_block = round_up((size_t)(4 * Qc * d->L * d->K), 64);
    const size_t table_plane = (size_t)(pl.nW * pl.t_stride) * sizeof(uint32_t);
    const size_t slab_plane = (size_t)(pl.nW * pl.slab_per_block) * sizeof(float4);
    auto bytes_for = [&](int64_t planes) {
        return round_up(kCountersBytes, kWorkspaceAlign) +
               round_up(table_plane * planes, kWorkspaceAlign) +
               round_up(slab_plane * planes, kWorkspaceAlign);
    };
    pl.min_bytes = bytes_for(1);
    int64_t per = BM;
    if (bytes_for(per) > budget) {
        if (pl.min_bytes > budget) return pl;   // bytes = 0: does not fit
        // the most planes that fit, rounded down to a multiple of 8 when >= 8
        int64_t lo = 1, hi = BM;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) / 2;
            if (bytes_for(mid) <= budget) lo = mid; else hi = mid - 1;
        }
        per = lo >= 8 ? lo - lo % 8 : lo;
    }
    pl.bm_per_pass = per;
    pl.passes = (BM + per - 1) / per;
    pl.counters_off = 0;
    pl.table_off = round_up(kCountersBytes, kWorkspaceAlign);   // after the 8 work counters
    pl.slab_off = pl.table_off + round_up(table_plane * per, kWorkspaceAlign);
    pl.bytes = bytes_for(per);
    return pl;
}

Params make_params(const msda_dims_t* d, msda_dtype_t dt, const void* value, const int64_t* shapes,
                   const int64_t* lsi, const float* loc, const float* attn) {
    Params p = {};
    p.value = value;
    p.shapes = shapes;
    p.lsi = lsi;
    p.loc = loc;
    p.attn = attn;
    p.B = (int)d->B;
    p.Nv = (int)d->Nv;
    p.M = (int)d->M;
    p.L = (int)d->L;
    p.Nq = (int)d->Nq;
    p.K = (int)d->K;
    p.LK = (int)(d->L * d->K);
    p.T = (int)(d->B * d->Nq * d->M);
    const int64_t elems = d->B * d->Nv * d->M * d->D;
    const int64_t elem = dt == MSDA_DTYPE_F32 ? 4 : 2;
    p.value_bytes = (uint32_t)(elems * elem);
    // heads whose value rows share a 128-byte line, taken together
    const int64_t per_line = 128 / (d->D * elem);
    p.hp = (per_line > 1 && d->M % per_line == 0) ? (int)per_line : 1;
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

// Blocks of the tile kernel that fit on one CU, asked of the runtime once per
// kernel and kept.
int tile_blocks_per_cu(int64_t D, const void* kernel, bool bf16_out, int tall) {
    static std::atomic<int> known[16];
    std::atomic<int>& slot =
        known[(D == 8 ? 0 : D == 16 ? 1 : D == 32 ? 2 : 3) + (bf16_out ? 4 : 0) + (tall ? 8 : 0)];
    int n = slot.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) != hipSuccess || n < 1) n = 1;
    slot.store(n, std::memory_order_relaxed);
    return n;
}

msda_status_t launch(const void* kernel, int64_t blocks, Params& p, hipStream_t stream) {
    if (blocks <= 0) return MSDA_SUCCESS;
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3(kBlock), args, 0, stream);
    return e == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_LAUNCH;
}

// Kernels of one (value type, D) instantiation.
struct Kernels {
    const void* fwd = nullptr;
    const void* point = nullptr;
    // bin kernels: [tall + 2 * cached]; tile kernels: [tall] (tall: tiles of
    // kTileHTall rows, else kTileH; cached: points kept in registers)
    const void* bin[4] = {};
    const void* tile[2] = {};
    const void* fwd_fused = nullptr;
    const void* point_fused = nullptr;
    const void* bin_fused[4] = {};
    const void* fwd_dcn = nullptr;
    const void* point_dcn = nullptr;
    const void* bin_dcn[4] = {};
    const void* fwd_half = nullptr;     // binary16 locations and weights
    const void* point_half = nullptr;
    const void* bin_half[4] = {};
    const void* tile_bf16[2] = {};      // grad_value stored as bf16
    // forward with the coarse levels in LDS, per front-end (null where
    // staged_row() rules the head's row width out)
    const void* fwd_staged = nullptr;
    const void* fwd_fused_staged = nullptr;
    const void* fwd_half_staged = nullptr;
    int head_bytes = 0;   // D * element size
    int tuples_per_block = 0;
};

template <typename T, int D>
Kernels kernels_for() {
    Kernels k;
    k.fwd = reinterpret_cast<const void*>(&msda_fwd_kernel<T, D, kFeCore>);
    k.point = reinterpret_cast<const void*>(&msda_bwd_point_kernel<T, D, kFeCore>);
    k.bin[0] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCore, kTileH, false>);
    k.bin[1] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCore, kTileHTall, false>);
    k.bin[2] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCore, kTileH, true>);
    k.bin[3] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCore, kTileHTall, true>);
    k.fwd_fused = reinterpret_cast<const void*>(&msda_fwd_kernel<T, D, kFeFused>);
    k.point_fused = reinterpret_cast<const void*>(&msda_bwd_point_kernel<T, D, kFeFused>);
    k.bin_fused[0] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeFused, kTileH, false>);
    k.bin_fused[1] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeFused, kTileHTall, false>);
    k.bin_fused[2] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeFused, kTileH, true>);
    k.bin_fused[3] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeFused, kTileHTall, true>);
    k.fwd_dcn = reinterpret_cast<const void*>(&msda_fwd_kernel<T, D, kFeDcn>);
    k.point_dcn = reinterpret_cast<const void*>(&msda_bwd_point_kernel<T, D, kFeDcn>);
    k.bin_dcn[0] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeDcn, kTileH, false>);
    k.bin_dcn[1] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeDcn, kTileHTall, false>);
    k.bin_dcn[2] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeDcn, kTileH, true>);
    k.bin_dcn[3] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeDcn, kTileHTall, true>);
    k.fwd_half = reinterpret_cast<const void*>(&msda_fwd_kernel<T, D, kFeCoreHalf>);
    k.point_half = reinterpret_cast<const void*>(&msda_bwd_point_kernel<T, D, kFeCoreHalf>);
    k.bin_half[0] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCoreHalf, kTileH, false>);
    k.bin_half[1] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCoreHalf, kTileHTall, false>);
    k.bin_half[2] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCoreHalf, kTileH, true>);
    k.bin_half[3] = reinterpret_cast<const void*>(&msda_bin_kernel<D, kFeCoreHalf, kTileHTall, true>);
    k.tile[0] = reinterpret_cast<const void*>(&msda_tile_kernel<D, false, kTileH>);
    k.tile[1] = reinterpret_cast<const void*>(&msda_tile_kernel<D, false, kTileHTall>);
    k.tile_bf16[0] = reinterpret_cast<const void*>(&msda_tile_kernel<D, true, kTileH>);
    k.tile_bf16[1] = reinterpret_cast<const void*>(&msda_tile_kernel<D, true, kTileHTall>);
    k.tuples_per_block = Shape<T, D>::TPW * kWavesPerBlock;
    k.head_bytes = D * Elem<T>::kBytes;
    if constexpr (staged_row(D * Elem<T>::kBytes)) {
        k.fwd_staged = reinterpret_cast<const void*>(&msda_fwd_staged_kernel<T, D, kFeCore>);
        k.fwd_fused_staged = reinterpret_cast<const void*>(&msda_fwd_staged_kernel<T, D, kFeFused>);
        k.fwd_half_staged =
            reinterpret_cast<const void*>(&msda_fwd_staged_kernel<T, D, kFeCoreHalf>);
    }
    return k;
}

// Whether the staged forward pays: planes of enough
// queries, and a coarsest level that fits in the stage. The level table is in
// device memory, so the host estimates the coarsest level's size from Nv and
// L as that of a pyramid that halves both sides from level to level
// (Nv = c (4^L - 1) / 3 for c pixels at the coarsest level). A wrong guess
// costs time, not correctness: the staged kernel stages what fits (possibly
// nothing) and reads every other level through buffer loads.
bool use_staged(const Params& p, int head_bytes) {
    if (!staged_row(head_bytes) || p.Nq < kStagedMinQueries || p.LK <= 0) return false;
    const double coarsest = 3.0 * (double)p.Nv / (std::ldexp(1.0, 2 * p.L) - 1.0);
    return (coarsest + 1.0) * head_bytes <= (double)kStageBytes;
}

// The forward of one front-end: the staged kernel where use_staged() says
// so, else the plain one.
msda_status_t launch_forward(const void* plain, const void* staged, const Kernels& k, Params& p,
                             hipStream_t stream) {
    if (staged && use_staged(p, k.head_bytes)) {
        const int64_t nqc = (p.Nq + kStagedQueries - 1) / kStagedQueries;
        const int64_t blocks = (int64_t)p.B * p.M * nqc;
        if (blocks <= 0) return MSDA_SUCCESS;
        void* args[] = {&p};
        const hipError_t e = hipLaunchKernel(staged, dim3((unsigned)blocks), dim3(kStagedBlock),
                                             args, 0, stream);
        return e == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_LAUNCH;
    }
    if (!plain) return MSDA_ERROR_NOT_SUPPORTED;
    return launch(plain, ((int64_t)p.T + k.tuples_per_block - 1) / k.tuples_per_block, p, stream);
}

Kernels pick(msda_dtype_t dt, int64_t D) {
#define MSDA_PICK(T, DD) \
    if (D == DD) return kernels_for<T, DD>();
    if (dt == MSDA_DTYPE_F32) {
        MSDA_PICK(float, 8) MSDA_PICK(float, 16) MSDA_PICK(float, 32) MSDA_PICK(float, 64)
    } else if (dt == MSDA_DTYPE_BF16) {
        MSDA_PICK(bf16_t, 8) MSDA_PICK(bf16_t, 16) MSDA_PICK(bf16_t, 32) MSDA_PICK(bf16_t, 64)
    } else if (dt == MSDA_DTYPE_F16) {
        MSDA_PICK(f16_t, 8) MSDA_PICK(f16_t, 16) MSDA_PICK(f16_t, 32) MSDA_PICK(f16_t, 64)
    }
#undef MSDA_PICK
    return Kernels();
}

// grad_value: the bin kernel, then the tile kernel, pass after pass, on the
// workspace of `pl` (bins and tiles hold the variants indexed as in Kernels;
// the plan picks).
msda_status_t launch_grad_value(Params& p, const BwdPlan& pl, const msda_dims_t* dims,
                                const void* const* bins, const void* const* tiles,
                                void* workspace, hipStream_t stream, bool bf16_out = false) {
    // the register-cached bin kernel holds kBinUnroll points per thread
    if (pl.cached && pl.Qc * dims->L * dims->K > (int64_t)kBinUnroll * kBlock)
        return MSDA_ERROR_LAUNCH;
    if (pl.bytes == 0 || pl.bm_per_pass < 1) return MSDA_ERROR_INVALID_VALUE;
    const void* bin = bins[pl.tall + 2 * pl.cached];
    const void* tile = tiles[pl.tall];
    p.nW = (int)pl.nW;
    p.Qc = (int)pl.Qc;
    p.t_stride = (int)pl.t_stride;
    p.slab_per_block = (uint32_t)pl.slab_per_block;
    p.table = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + pl.table_off);
    p.slab = reinterpret_cast<float4*>(static_cast<char*>(workspace) + pl.slab_off);
    p.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + pl.counters_off);
    p.grad_value_bytes =
        (uint32_t)(dims->B * dims->Nv * dims->M * dims->D * (bf16_out ? 2 : 4));   // < 2 GiB
    // persistent tile kernel: blocks fetch (b, m, tile) work items, as many
    // blocks as fit on the GPU at once; the grid is a multiple of 8 for the
    // XCD-affine schedule
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MSDA_ERROR_LAUNCH;
    const int per_cu = tile_blocks_per_cu(dims->D, tile, bf16_out, pl.tall);
    const int64_t resident = ((int64_t)per_cu * (cus > 0 ? cus : 1) + 7) / 8 * 8;
    const int64_t BM = dims->B * dims->M;
    for (int64_t bm0 = 0; bm0 < BM; bm0 += pl.bm_per_pass) {
        p.bm0 = (int)bm0;
        p.bm_count = (int)std::min<int64_t>(pl.bm_per_pass, BM - bm0);
        // a pass whose entries (about one 16-byte entry per point) outgrow
        // the eight 4 MB L2s writes them non-temporal (encoder_train: 182 MB,
        // grad_value stage 284 -> 266 us); a small one keeps them in the L2
        // for the tile kernel (the 300-query decoder: 4.9 MB, 3 us faster)
        p.slab_streaming =
            (int64_t)p.bm_count * dims->Nq * dims->L * dims->K * 16 > ((int64_t)32 << 20);
        msda_status_t s = launch(bin, p.bm_count * pl.nW, p, stream);
        if (s != MSDA_SUCCESS) return s;
        const int64_t items = p.bm_count * (pl.t_stride - 1);
        const int64_t grid = items < resident ? ((items + 7) / 8) * 8 : resident;
        s = launch(tile, grid, p, stream);
        if (s != MSDA_SUCCESS) return s;
    }
    return MSDA_SUCCESS;
}

// Workspace of the fused backward: the tuples' softmax statistics, room for
// the offsets' gradient when the caller asks for the reference points'
// gradient only, then the core's grad_value workspace (planned for what is
// left of `budget`).
struct FusedPlan {
    BwdPlan core;
    size_t smax_off = 0, goff_off = 0, core_off = 0, bytes = 0;
};

FusedPlan plan_backward_fused(const msda_dims_t* d, size_t budget = SIZE_MAX) {
    FusedPlan f;
    const Sizes n = sizes_of(d);
    const int64_t T = d->B * d->Nq * d->M;
    f.smax_off = 0;
    f.goff_off = round_up((size_t)T * sizeof(float2), kWorkspaceAlign);
    f.core_off = f.goff_off + round_up((size_t)n.points * 2 * sizeof(float), kWorkspaceAlign);
    f.core = plan_backward(d, budget > f.core_off ? budget - f.core_off : 0);
    f.bytes = f.core_off + f.core.bytes;
    return f;
}

msda_status_t check_precision(const msda_precision_t* pr) {
    if (!pr) return MSDA_ERROR_INVALID_VALUE;
    if (pr->value != MSDA_DTYPE_F32 && pr->value != MSDA_DTYPE_BF16 && pr->value != MSDA_DTYPE_F16)
        return MSDA_ERROR_INVALID_VALUE;
    if (pr->locations != MSDA_DTYPE_F32 && pr->locations != MSDA_DTYPE_F16)
        return MSDA_ERROR_INVALID_VALUE;
    if (pr->grad_value != MSDA_DTYPE_F32 && pr->grad_value != MSDA_DTYPE_BF16)
        return MSDA_ERROR_INVALID_VALUE;
    return MSDA_SUCCESS;
}

msda_status_t forward_impl(const msda_dims_t* dims, const msda_precision_t& pr, const void* value,
                           const int64_t* spatial_shapes, const int64_t* level_start_index,
                           const void* sampling_locations, const void* attention_weights,
                           float* output, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, pr.value, false);
    if (st != MSDA_SUCCESS) return st;
    const bool half = pr.locations == MSDA_DTYPE_F16;
    const Sizes n = sizes_of(dims);
    // a tensor with no elements may come as NULL
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_locations || !attention_weights)) || (n.out && !output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(output, 16) || !aligned(sampling_locations, half ? 4 : 8) ||
        !aligned(attention_weights, half ? 2 : 4) || !aligned(spatial_shapes, 8) ||
        !aligned(level_start_index, 8))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, pr.value, value, spatial_shapes, level_start_index,
                           static_cast<const float*>(sampling_locations),
                           static_cast<const float*>(attention_weights));
    p.out = output;
    if (p.T == 0) return MSDA_SUCCESS;
    const Kernels k = pick(pr.value, dims->D);
    return launch_forward(half ? k.fwd_half : k.fwd, half ? k.fwd_half_staged : k.fwd_staged, k, p,
                          stream);
}

msda_status_t backward_impl(const msda_dims_t* dims, const msda_precision_t& pr, const void* value,
                            const int64_t* spatial_shapes, const int64_t* level_start_index,
                            const void* sampling_locations, const void* attention_weights,
                            const float* grad_output, void* grad_value,
                            float* grad_sampling_locations, float* grad_attention_weights,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, pr.value, true);
    if (st != MSDA_SUCCESS) return st;
    const bool half = pr.locations == MSDA_DTYPE_F16;
    const bool bf16_out = pr.grad_value == MSDA_DTYPE_BF16;
    const Sizes n = sizes_of(dims);
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_locations || !attention_weights)) || (n.out && !grad_output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(grad_output, 16) || !aligned(grad_value, 16) ||
        !aligned(sampling_locations, half ? 4 : 8) || !aligned(grad_sampling_locations, 8) ||
        !aligned(attention_weights, half ? 2 : 4) || !aligned(grad_attention_weights, 4) ||
        !aligned(spatial_shapes, 8) || !aligned(level_start_index, 8) ||
        !aligned(workspace, kWorkspaceAlign))
        return MSDA_ERROR_INVALID_VALUE;
    const BwdPlan pl = plan_backward(dims, workspace ? workspace_bytes : 0);
    if (grad_value && n.value && (!workspace || pl.bytes == 0)) return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, pr.value, value, spatial_shapes, level_start_index,
                           static_cast<const float*>(sampling_locations),
                           static_cast<const float*>(attention_weights));
    p.grad_out = grad_output;
    p.grad_value = static_cast<float*>(grad_value);
    p.grad_loc = grad_sampling_locations;
    p.grad_attn = grad_attention_weights;
    const Kernels k = pick(pr.value, dims->D);
    const void* point = half ? k.point_half : k.point;
    if (!point) return MSDA_ERROR_NOT_SUPPORTED;
    if (grad_value && n.value) {
        const msda_status_t s =
            launch_grad_value(p, pl, dims, half ? k.bin_half : k.bin,
                              bf16_out ? k.tile_bf16 : k.tile, workspace, stream, bf16_out);
        if (s != MSDA_SUCCESS) return s;
    }
    if (p.T == 0 || (!grad_sampling_locations && !grad_attention_weights)) return MSDA_SUCCESS;
    return launch(point, ((int64_t)p.T + k.tuples_per_block - 1) / k.tuples_per_block, p, stream);
}

}  // namespace

extern "C" {

msda_status_t msda_forward(const msda_dims_t* dims, msda_dtype_t value_dtype, const void* value,
                           const int64_t* spatial_shapes, const int64_t* level_start_index,
                           const float* sampling_locations, const float* attention_weights,
                           float* output, hipStream_t stream) {
    const msda_precision_t pr = {value_dtype, MSDA_DTYPE_F32, MSDA_DTYPE_F32};
    return forward_impl(dims, pr, value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights, output, stream);
}

msda_status_t msda_forward_ex(const msda_dims_t* dims, const msda_precision_t* precision,
                              const void* value, const int64_t* spatial_shapes,
                              const int64_t* level_start_index, const void* sampling_locations,
                              const void* attention_weights, float* output, hipStream_t stream) {
    const msda_status_t st = check_precision(precision);
    if (st != MSDA_SUCCESS) return st;
    return forward_impl(dims, *precision, value, spatial_shapes, level_start_index,
                        sampling_locations, attention_weights, output, stream);
}

msda_status_t msda_backward_workspace_size(const msda_dims_t* dims, msda_dtype_t value_dtype,
                                           size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    *bytes = plan_backward(dims).bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_backward_workspace_min_size(const msda_dims_t* dims, msda_dtype_t value_dtype,
                                               size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    *bytes = plan_backward(dims).min_bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_backward(const msda_dims_t* dims, msda_dtype_t value_dtype, const void* value,
                            const int64_t* spatial_shapes, const int64_t* level_start_index,
                            const float* sampling_locations, const float* attention_weights,
                            const float* grad_output, float* grad_value,
                            float* grad_sampling_locations, float* grad_attention_weights,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const msda_precision_t pr = {value_dtype, MSDA_DTYPE_F32, MSDA_DTYPE_F32};
    return backward_impl(dims, pr, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_output, grad_value, grad_sampling_locations,
                         grad_attention_weights, workspace, workspace_bytes, stream);
}

msda_status_t msda_backward_ex(const msda_dims_t* dims, const msda_precision_t* precision,
                               const void* value, const int64_t* spatial_shapes,
                               const int64_t* level_start_index, const void* sampling_locations,
                               const void* attention_weights, const float* grad_output,
                               void* grad_value, float* grad_sampling_locations,
                               float* grad_attention_weights, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    const msda_status_t st = check_precision(precision);
    if (st != MSDA_SUCCESS) return st;
    return backward_impl(dims, *precision, value, spatial_shapes, level_start_index,
                         sampling_locations, attention_weights, grad_output, grad_value,
                         grad_sampling_locations, grad_attention_weights, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free backward
// The scratch of msda_backward_noalloc: a static device array, one copy per GPU
// (reserved when the code object is loaded on that GPU, held until the process
// ends). In host code `scratch` names a host-side stand-in, not device memory:
// kernels and copies get the device address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[MSDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// This device's copy of `scratch`, looked up on the first call on the device
// (with the device current); nullptr if the runtime cannot give it.
void* noalloc_scratch(int dev) {
    static std::atomic<void*> known[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = known[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    known[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

extern "C" {

msda_status_t msda_backward_noalloc(const msda_dims_t* dims, msda_dtype_t value_dtype,
                                    const void* value, const int64_t* spatial_shapes,
                                    const int64_t* level_start_index,
                                    const float* sampling_locations,
                                    const float* attention_weights, const float* grad_output,
                                    float* grad_value, float* grad_sampling_locations,
                                    float* grad_attention_weights, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (grad_value && sizes_of(dims).value > 0) {
        // as many (b, m) planes per pass as the scratch holds
        if (plan_backward(dims, MSDA_NOALLOC_SCRATCH_BYTES).bytes == 0)
            return MSDA_ERROR_SCRATCH_TOO_SMALL;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MSDA_ERROR_LAUNCH;
        ws = noalloc_scratch(dev);
        if (!ws) return MSDA_ERROR_LAUNCH;
        ws_bytes = MSDA_NOALLOC_SCRATCH_BYTES;
    }
    const msda_precision_t pr = {value_dtype, MSDA_DTYPE_F32, MSDA_DTYPE_F32};
    return backward_impl(dims, pr, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_weights, grad_output, grad_value, grad_sampling_locations,
                         grad_attention_weights, ws, ws_bytes, stream);
}

msda_status_t msda_forward_fused(const msda_dims_t* dims, msda_dtype_t value_dtype,
                                 const void* value, const int64_t* spatial_shapes,
                                 const int64_t* level_start_index, const float* reference_points,
                                 const float* sampling_offsets, const float* attention_logits,
                                 float* output, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, value_dtype, false);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(dims);
    const int64_t n_ref = dims->B * dims->Nq * dims->L * 2;
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_offsets || !attention_logits)) || (n_ref && !reference_points) ||
        (n.out && !output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(output, 16) || !aligned(sampling_offsets, 8) ||
        !aligned(reference_points, 8) || !aligned(attention_logits, 4) ||
        !aligned(spatial_shapes, 8) || !aligned(level_start_index, 8))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, value_dtype, value, spatial_shapes, level_start_index, nullptr,
                           nullptr);
    p.ref = reference_points;
    p.off = sampling_offsets;
    p.logits = attention_logits;
    p.out = output;
    if (p.T == 0) return MSDA_SUCCESS;
    const Kernels k = pick(value_dtype, dims->D);
    return launch_forward(k.fwd_fused, k.fwd_fused_staged, k, p, stream);
}

msda_status_t msda_backward_fused_workspace_size(const msda_dims_t* dims,
                                                 msda_dtype_t value_dtype, size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    *bytes = plan_backward_fused(dims).bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_backward_fused(const msda_dims_t* dims, msda_dtype_t value_dtype,
                                  const void* value, const int64_t* spatial_shapes,
                                  const int64_t* level_start_index, const float* reference_points,
                                  const float* sampling_offsets, const float* attention_logits,
                                  const float* grad_output, float* grad_value,
                                  float* grad_reference_points, float* grad_sampling_offsets,
                                  float* grad_attention_logits, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    const msda_status_t st = check_dims(dims, value_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(dims);
    const int64_t n_ref = dims->B * dims->Nq * dims->L * 2;
    if ((n.value && !value) || !spatial_shapes || !level_start_index ||
        (n.points && (!sampling_offsets || !attention_logits)) || (n_ref && !reference_points) ||
        (n.out && !grad_output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, 16) || !aligned(grad_output, 16) || !aligned(grad_value, 16) ||
        !aligned(sampling_offsets, 8) || !aligned(grad_sampling_offsets, 8) ||
        !aligned(reference_points, 8) || !aligned(grad_reference_points, 8) ||
        !aligned(attention_logits, 4) || !aligned(grad_attention_logits, 4) ||
        !aligned(spatial_shapes, 8) || !aligned(level_start_index, 8) ||
        !aligned(workspace, kWorkspaceAlign))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(dims, value_dtype, value, spatial_shapes, level_start_index, nullptr,
                           nullptr);
    const bool want_value = grad_value && n.value;
    const bool want_point =
        p.T > 0 && (grad_reference_points || grad_sampling_offsets || grad_attention_logits);
    if (!want_value && !want_point) return MSDA_SUCCESS;
    const FusedPlan pl = plan_backward_fused(dims, workspace ? workspace_bytes : 0);
    if (!workspace || workspace_bytes < pl.core_off || (want_value && pl.core.bytes == 0))
        return MSDA_ERROR_INVALID_VALUE;
    p.ref = reference_points;
    p.off = sampling_offsets;
    p.logits = attention_logits;
    p.grad_out = grad_output;
    p.grad_value = grad_value;
    p.smax = reinterpret_cast<float2*>(static_cast<char*>(workspace) + pl.smax_off);
    const Kernels k = pick(value_dtype, dims->D);
    if (!k.point_fused) return MSDA_ERROR_NOT_SUPPORTED;
    // (none if T = 0; at most 2^20 blocks, which stride over the tuples)
    msda_status_t s = launch(reinterpret_cast<const void*>(&msda_softmax_stats_kernel),
                             std::min<int64_t>((4 * (int64_t)p.T + kBlock - 1) / kBlock, 1 << 20),
                             p, stream);
    if (s != MSDA_SUCCESS) return s;
    if (want_value) {
        s = launch_grad_value(p, pl.core, dims, k.bin_fused, k.tile,
                              static_cast<char*>(workspace) + pl.core_off, stream);
        if (s != MSDA_SUCCESS) return s;
    }
    if (!want_point) return MSDA_SUCCESS;
    p.grad_off = grad_sampling_offsets
                     ? grad_sampling_offsets
                     : (grad_reference_points
                            ? reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.goff_off)
                            : nullptr);
    p.grad_logits = grad_attention_logits;
    s = launch(k.point_fused, ((int64_t)p.T + k.tuples_per_block - 1) / k.tuples_per_block, p,
               stream);
    if (s != MSDA_SUCCESS || !grad_reference_points) return s;
    const int64_t nref = dims->B * dims->Nq * dims->L;
    void* args[] = {&p, &grad_reference_points};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&msda_ref_grad_kernel),
                                         dim3((unsigned)((nref + kBlock - 1) / kBlock)), dim3(kBlock),
                                         args, 0, stream);
    return e == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_LAUNCH;
}

}  // extern "C"

namespace {

// The grouped single-level problem as a core problem: one level of H x W
// pixels, G heads of D channels, the H_out x W_out output pixels as queries
// and the kernel_h x kernel_w grid points as the points of that level.
msda_status_t dcn_dims(const msda_dcn_dims_t* d, msda_dims_t* o) {
    if (!d) return MSDA_ERROR_INVALID_VALUE;
    if (d->B < 0 || d->H < 1 || d->W < 1 || d->G < 1 || d->D < 1 || d->kernel_h < 1 ||
        d->kernel_w < 1 || d->stride_h < 1 || d->stride_w < 1 || d->pad_h < 0 || d->pad_w < 0 ||
        d->dilation_h < 1 || d->dilation_w < 1 || d->H_out < 0 || d->W_out < 0)
        return MSDA_ERROR_INVALID_VALUE;
    // grid coordinates stay exact in fp32 and in 32-bit integers
    const int64_t lim = (int64_t)1 << 24;
    if (d->H >= lim || d->W >= lim || d->H_out >= lim || d->W_out >= lim ||
        d->kernel_h >= lim || d->kernel_w >= lim || d->kernel_h * d->kernel_w >= lim ||
        d->H_out * d->stride_h + d->pad_h + d->kernel_h * d->dilation_h >= lim ||
        d->W_out * d->stride_w + d->pad_w + d->kernel_w * d->dilation_w >= lim)
        return MSDA_ERROR_NOT_SUPPORTED;
    o->B = d->B;
    o->Nv = d->H * d->W;
    o->M = d->G;
    o->D = d->D;
    o->L = 1;
    o->Nq = d->H_out * d->W_out;
    o->K = d->kernel_h * d->kernel_w;
    return MSDA_SUCCESS;
}

void dcn_params(Params& p, const msda_dcn_dims_t* d) {
    p.shapes = nullptr;
    p.lsi = nullptr;
    p.lvl_H = (int)d->H;
    p.lvl_W = (int)d->W;
    p.out_W = (int)std::max<int64_t>(d->W_out, 1);
    p.kernel_w = (int)d->kernel_w;
    p.stride_h = (int)d->stride_h;
    p.stride_w = (int)d->stride_w;
    p.pad_h = (int)d->pad_h;
    p.pad_w = (int)d->pad_w;
    p.dil_h = (int)d->dilation_h;
    p.dil_w = (int)d->dilation_w;
}

}  // namespace

extern "C" {

msda_status_t msda_dcn_forward(const msda_dcn_dims_t* dcn, msda_dtype_t input_dtype,
                               const void* input, const float* offset, const float* mask,
                               float* output, hipStream_t stream) {
    msda_dims_t dims;
    msda_status_t st = dcn_dims(dcn, &dims);
    if (st != MSDA_SUCCESS) return st;
    st = check_dims(&dims, input_dtype, false);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(&dims);
    if ((n.value && !input) || (n.points && (!offset || !mask)) || (n.out && !output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(input, 16) || !aligned(output, 16) || !aligned(offset, 8) || !aligned(mask, 4))
        return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(&dims, input_dtype, input, nullptr, nullptr, nullptr, mask);
    dcn_params(p, dcn);
    p.off = offset;
    p.out = output;
    if (p.T == 0) return MSDA_SUCCESS;
    const Kernels k = pick(input_dtype, dims.D);
    if (!k.fwd_dcn) return MSDA_ERROR_NOT_SUPPORTED;
    return launch(k.fwd_dcn, ((int64_t)p.T + k.tuples_per_block - 1) / k.tuples_per_block, p,
                  stream);
}

msda_status_t msda_dcn_backward_workspace_size(const msda_dcn_dims_t* dcn,
                                               msda_dtype_t input_dtype, size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    msda_dims_t dims;
    msda_status_t st = dcn_dims(dcn, &dims);
    if (st != MSDA_SUCCESS) return st;
    st = check_dims(&dims, input_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    *bytes = plan_backward(&dims).bytes;
    return MSDA_SUCCESS;
}

msda_status_t msda_dcn_backward(const msda_dcn_dims_t* dcn, msda_dtype_t input_dtype,
                                const void* input, const float* offset, const float* mask,
                                const float* grad_output, float* grad_input, float* grad_offset,
                                float* grad_mask, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    msda_dims_t dims;
    msda_status_t st = dcn_dims(dcn, &dims);
    if (st != MSDA_SUCCESS) return st;
    st = check_dims(&dims, input_dtype, true);
    if (st != MSDA_SUCCESS) return st;
    const Sizes n = sizes_of(&dims);
    if ((n.value && !input) || (n.points && (!offset || !mask)) || (n.out && !grad_output))
        return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(input, 16) || !aligned(grad_output, 16) || !aligned(grad_input, 16) ||
        !aligned(offset, 8) || !aligned(grad_offset, 8) || !aligned(mask, 4) ||
        !aligned(grad_mask, 4) || !aligned(workspace, kWorkspaceAlign))
        return MSDA_ERROR_INVALID_VALUE;
    const BwdPlan pl = plan_backward(&dims, workspace ? workspace_bytes : 0);
    if (grad_input && n.value && (!workspace || pl.bytes == 0)) return MSDA_ERROR_INVALID_VALUE;
    Params p = make_params(&dims, input_dtype, input, nullptr, nullptr, nullptr, mask);
    dcn_params(p, dcn);
    p.off = offset;
    p.grad_out = grad_output;
    p.grad_value = grad_input;
    p.grad_off = grad_offset;
    p.grad_attn = grad_mask;
    const Kernels k = pick(input_dtype, dims.D);
    if (!k.point_dcn) return MSDA_ERROR_NOT_SUPPORTED;
    if (grad_input && n.value) {
        st = launch_grad_value(p, pl, &dims, k.bin_dcn, k.tile, workspace, stream);
        if (st != MSDA_SUCCESS) return st;
    }
    if (p.T == 0 || (!grad_offset && !grad_mask)) return MSDA_SUCCESS;
    return launch(k.point_dcn, ((int64_t)p.T + k.tuples_per_block - 1) / k.tuples_per_block, p,
                  stream);
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
        case MSDA_ERROR_INVALID_VALUE: return "invalid value (pointer, alignment, size or workspace)";
        case MSDA_ERROR_NOT_SUPPORTED: return "not supported (D, level count or tensor size)";
        case MSDA_ERROR_LAUNCH: return "kernel launch failed";
        case MSDA_ERROR_SCRATCH_TOO_SMALL:
            return "the problem needs more scratch than the allocation-free backward holds "
                   "(use msda_backward with a workspace)";
    }
    return "unknown status";
}

int msda_version(void) {
    return MSDA_VERSION_MAJOR * 10000 + MSDA_VERSION_MINOR * 100 + MSDA_VERSION_PATCH;
}

}  // extern "C"
