// linear.hip -- the fully connected projections around the deformable
// attention core on the gfx950 matrix cores: y = x W^T + b and its gradients
// (torch nn.Linear semantics). In MSDeformAttn four of them surround the core:
// the value projection, the sampling-offset and attention-weight heads on the
// query, and the output projection (deformable-attention tutorial (discosf.com),
// section 3.1; DETR-to-Deformable-DETR article, section 3.2).
//
// One kernel serves the three products a linear layer needs:
//   forward      y[r, o]  = sum_i x[r, i] W[o, i]       (both operands i-contiguous)
//   input grad   dx[r, i] = sum_o dy[r, o] W[o, i]      (W walked along its rows)
//   weight grad  dW[o, i] = sum_r dy[r, o] x[r, i]      (reduction over the rows,
//                                                         split over blocks)
// Block tile 128 x 128, four waves of 64 x 64, each a 2 x 2 grid of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, fed with three-term bf16
// splits of the fp32 operands (six products per fp32 product, fp32 accuracy;
// see msda_gemm_kernel). A 16-deep slice of both operands is staged in LDS,
// split on the way, double buffered; while a slice feeds the matrix cores the
// next slice's weight-side operand and the A operand two slices ahead are in
// flight (A streams from HBM; B is mostly small and L2-resident).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gemm.h"
#include "msda.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;          // 4 waves
constexpr int kTile = 128;             // block tile, rows and columns
constexpr int kBK = 16;                // reduction slice per iteration (one MFMA step)
constexpr int kPerThread = kTile * kBK / 256;   // staged elements of an operand per thread
constexpr int kSplitMax = 256;         // reduction splits of a weight gradient at most

// C = A B (+ bias) (+ C) with A(m, k), B(k, n) read through strides:
//   kAK: A(m, k) = A[m * lda + k]   else A[k * lda + m]
//   kBK_: B(k, n) = B[n * ldb + k]  else B[k * ldb + n]
struct GemmArgs {
    const float* A;
    const float* B;
    float* C;
    const float* bias;     // [N], or null
    int64_t lda, ldb, ldc;
    int M, N, K;
    int k_split;           // reduction length per split (a multiple of kBK)
    int splits;
    int accumulate;        // C += result (splits == 1 only)
    int64_t split_stride;  // elements between consecutive splits' partial outputs
    float* asum;           // if set: sum over this split's k of A(m, k), at asum[z * M + m]
    // optional second reduction segment, k in [K, K + K2): A2, B2 with the
    // same layouts (K a multiple of kBK, so a slice never straddles)
    const float* A2;
    const float* B2;
    int64_t lda2, ldb2;
    int K2;
    int unit_begin;        // first work item of this problem in its group
};

// Up to kMaxGroup independent products of one operand-layout combination in
// one launch: the work items of all of them share the grid, so the last
// partial round of blocks is paid once.
constexpr int kMaxGroup = 4;
struct GemmGroup {
    GemmArgs g[kMaxGroup];
    int count;
};

// Blocks are dealt to the 8 XCDs round-robin; give each XCD a contiguous
// range of work items so that the column tiles of one row tile (which share
// the rows of A) meet in one L2.
__device__ inline int xcd_work_item() {
    const int blk = blockIdx.x, nblk = gridDim.x;
    const int x = blk % 8, i = blk / 8, per = nblk / 8, rem = nblk % 8;
    return x * per + (x < rem ? x : rem) + i;
}

// The products on the bf16 matrix cores, to fp32 accuracy: every fp32
// operand element x is split into three bf16 terms, x1 = bf16(x),
// x2 = bf16(x - x1), x3 = bf16(x - x1 - x2) (round to nearest even; the
// differences are exact in fp32), which carry x's 24 significant bits, and
// a b is summed as the six products whose terms' orders add to at most 4:
//   a1 b1 + a1 b2 + a2 b1 + a1 b3 + a2 b2 + a3 b1.
// Each term keeps the remainder of the previous ones to within 2^-8 of it,
// so |a - a1 - a2 - a3| <= 2^-24 |a|; the three dropped products and the two
// remainders add up to less than 2^-22 |a b| (four fp32 unit roundings), and
// every bf16 x bf16 product is exact in the fp32 accumulator, so the result
// carries the error of an fp32 product sum, within a small factor. v_mfma_f32_32x32x16_bf16 runs at 16 times the fp32
// rate, so the six products cost 3/8 of one fp32 product. A non-finite
// operand element yields NaN in the rows and columns it feeds.
//
// LDS: per operand and buffer, three planes of kTile rows x 16 k (bf16,
// 32 bytes a row); the two 16-byte halves of a row swap places on every
// second group of 8 rows, so that the fragment reads (one half-row per lane,
// rows 0..31 of a tile) hit distinct banks.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kSplitBK = kBK;                      // reduction slice (one MFMA step)
constexpr int kPlane = kTile * kSplitBK;           // bf16 elements of one plane

__device__ inline int swz(int row, int k) {      // element offset of (row, k) in a plane
    return row * kSplitBK + ((((k >> 3) ^ (row >> 3)) & 1) << 3) + (k & 7);
}

__device__ inline void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
    h = (__bf16)x;
    const float r1 = x - (float)h;
    m = (__bf16)r1;
    l = (__bf16)(r1 - (float)m);
}

template <bool kAK, bool kBKm, bool kVec>
__global__ __launch_bounds__(kThreads) void msda_gemm_kernel(GemmGroup grp) {
    __shared__ __attribute__((aligned(16))) __bf16 As[2][3 * kPlane];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][3 * kPlane];
    const int tid = threadIdx.x;
    const int work = xcd_work_item();
    int pi = 0;
    while (pi + 1 < grp.count && work >= grp.g[pi + 1].unit_begin) ++pi;
    const GemmArgs& g = grp.g[pi];
    const int local = work - g.unit_begin;
    const int mt = (g.M + kTile - 1) / kTile, nt = (g.N + kTile - 1) / kTile;
    const int z = local / (mt * nt);
    const int t = local - z * (mt * nt);
    const int m0 = (t / nt) * kTile, n0 = (t % nt) * kTile;
    const int kbeg = z * g.k_split;
    const int kend = min(g.K + g.K2, kbeg + g.k_split);

    // ---- staging: kTile * kSplitBK elements of each operand per slice; each
    // thread takes groups of four consecutive k of one row (a float4 when the
    // operand is k-contiguous, else four loads that the wave's lanes, on
    // consecutive rows, read coalesced) and writes each group split into the
    // three planes, 8 bytes per plane
    float ra[kPerThread], rb[kPerThread];
    auto group = [&](bool kmajor, int i, int& mn, int& k) {
        const int idx = tid + kThreads * i;
        if (kmajor) {
            mn = idx / (kSplitBK / 4);
            k = (idx % (kSplitBK / 4)) * 4;
        } else {
            mn = idx % kTile;
            k = (idx / kTile) * 4;
        }
    };
    auto load = [&](const float* P, int64_t ld, bool kmajor, int lim_mn, int base_mn, int k0,
                    int kend, float* r) {
        if constexpr (kVec) {
#pragma unroll
            for (int i = 0; i < kPerThread / 4; ++i) {
                int mn, k;
                group(kmajor, i, mn, k);
                const bool row_ok = base_mn + mn < lim_mn;
                if (kmajor) {
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (row_ok && k0 + k < kend)
                        v = *reinterpret_cast<const float4*>(P + (int64_t)(base_mn + mn) * ld +
                                                             (k0 + k));
                    r[4 * i] = v.x;
                    r[4 * i + 1] = v.y;
                    r[4 * i + 2] = v.z;
                    r[4 * i + 3] = v.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r[4 * i + e] = row_ok && k0 + k + e < kend
                                           ? P[(int64_t)(k0 + k + e) * ld + (base_mn + mn)]
                                           : 0.0f;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int idx = tid + kThreads * i;
                const int mn = kmajor ? idx / kSplitBK : idx % kTile;
                const int k = kmajor ? idx % kSplitBK : idx / kTile;
                const bool ok = base_mn + mn < lim_mn && k0 + k < kend;
                r[i] = ok ? (kmajor ? P[(int64_t)(base_mn + mn) * ld + (k0 + k)]
                                    : P[(int64_t)(k0 + k) * ld + (base_mn + mn)])
                          : 0.0f;
            }
        }
    };
    auto store = [&](__bf16* S, bool kmajor, const float* r) {
        if constexpr (kVec) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int i = 0; i < kPerThread / 4; ++i) {
                int mn, k;
                group(kmajor, i, mn, k);
                __bf16 h[4], m[4], l[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split3(r[4 * i + e], h[e], m[e], l[e]);
                const int o = swz(mn, k);
                *reinterpret_cast<bf16x4*>(&S[o]) = bf16x4{h[0], h[1], h[2], h[3]};
                *reinterpret_cast<bf16x4*>(&S[kPlane + o]) = bf16x4{m[0], m[1], m[2], m[3]};
                *reinterpret_cast<bf16x4*>(&S[2 * kPlane + o]) = bf16x4{l[0], l[1], l[2], l[3]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const int idx = tid + kThreads * i;
                const int mn = kmajor ? idx / kSplitBK : idx % kTile;
                const int k = kmajor ? idx % kSplitBK : idx / kTile;
                __bf16 h, m, l;
                split3(r[i], h, m, l);
                const int o = swz(mn, k);
                S[o] = h;
                S[kPlane + o] = m;
                S[2 * kPlane + o] = l;
            }
        }
    };

    // ---- wave tile 64 x 64 at (wm, wn); lane (li, lk) feeds row/column li
    // with k = 8 lk .. 8 lk + 7 of the slice
    const int lane = tid & 63, w = tid >> 6;
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
    const int li = lane & 31, lk = lane >> 5;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // column sums of A (a bias gradient rides along with its weight
    // gradient): with A not k-contiguous (the weight gradient's dy^T) the
    // fp32 values are summed as staged -- rows tid % kTile, two threads per
    // row, combined at the end; otherwise from the planes, one thread per row
    constexpr bool kAsumStaged = kVec && !kAK;
    const bool do_asum = g.asum != nullptr && n0 == 0 && (kAsumStaged || tid < kTile);
    float asum = 0.0f;

    auto fetchA = [&](int k0, float* r) {
        if (k0 >= g.K) load(g.A2, g.lda2, kAK, g.M, m0, k0 - g.K, kend - g.K, r);
        else load(g.A, g.lda, kAK, g.M, m0, k0, min(kend, g.K), r);
    };
    auto fetchB = [&](int k0) {
        if (k0 >= g.K) load(g.B2, g.ldb2, kBKm, g.N, n0, k0 - g.K, kend - g.K, rb);
        else load(g.B, g.ldb, kBKm, g.N, n0, k0, min(kend, g.K), rb);
    };
    float ra2[kPerThread];   // A two slices ahead

    auto asum_staged = [&]() {
        if constexpr (kAsumStaged) {
            if (do_asum) {
#pragma unroll
                for (int i = 0; i < kPerThread; ++i) asum += ra[i];
            }
        }
    };
    int buf = 0;
    if (kbeg < kend) {
        fetchA(kbeg, ra);
        fetchB(kbeg);
        asum_staged();
        store(As[0], kAK, ra);
        store(Bs[0], kBKm, rb);
        if (kbeg + kSplitBK < kend) fetchA(kbeg + kSplitBK, ra);
    }
    __syncthreads();
    for (int k0 = kbeg; k0 < kend; k0 += kSplitBK) {
        const bool more = k0 + kSplitBK < kend;
        if (more) fetchB(k0 + kSplitBK);
        if (k0 + 2 * kSplitBK < kend) fetchA(k0 + 2 * kSplitBK, ra2);
        const __bf16* Ab = As[buf];
        const __bf16* Bb = Bs[buf];
        bf16x8 fa[2][3], fb[2][3];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const int ar = wm + 32 * t2 + li, br = wn + 32 * t2 + li;
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                fa[t2][q] = *reinterpret_cast<const bf16x8*>(&Ab[q * kPlane + swz(ar, 8 * lk)]);
                fb[t2][q] = *reinterpret_cast<const bf16x8*>(&Bb[q * kPlane + swz(br, 8 * lk)]);
            }
        }
        // the six products, each over the four tiles in turn (independent
        // accumulators between dependent steps)
        constexpr int kPa[6] = {0, 0, 1, 0, 1, 2};
        constexpr int kPb[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
        for (int pr = 0; pr < 6; ++pr) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][kPa[pr]],
                                                                         fb[b][kPb[pr]],
                                                                         acc[a][b], 0, 0, 0);
        }
        if constexpr (!kAsumStaged) {
            if (do_asum) {
#pragma unroll
                for (int q = 0; q < kSplitBK; ++q) {
                    const int o = swz(tid, q);
                    asum += ((float)Ab[o] + (float)Ab[kPlane + o]) + (float)Ab[2 * kPlane + o];
                }
            }
        }
        if (more) {
            asum_staged();
            store(As[buf ^ 1], kAK, ra);
            store(Bs[buf ^ 1], kBKm, rb);
        }
        __syncthreads();
        buf ^= 1;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) ra[i] = ra2[i];
    }

    if constexpr (kAsumStaged) {
        if (g.asum != nullptr && n0 == 0) {   // block-uniform
            float* red = reinterpret_cast<float*>(As[0]);   // free after the last barrier
            red[tid] = asum;
            __syncthreads();
            if (tid < kTile && m0 + tid < g.M)
                g.asum[(int64_t)z * g.M + m0 + tid] = red[tid] + red[tid + kTile];
        }
    } else {
        if (do_asum && m0 + tid < g.M) g.asum[(int64_t)z * g.M + m0 + tid] = asum;
    }

    // ---- epilogue: 32x32 accumulator register r of lane (li, lk) holds
    // row 8 * (r / 4) + 4 * lk + r % 4, column li
    float* C = g.C + (int64_t)z * g.split_stride;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn + 32 * b + li;
            if (col >= g.N) continue;
            const float bv = g.bias ? g.bias[col] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * a + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (row < g.M) {
                    float* dst = C + (int64_t)row * g.ldc + col;
                    float v = acc[a][b][r] + bv;
                    if (g.accumulate) v += *dst;
                    *dst = v;
                }
            }
        }
    }
}


// out[m, n] (row stride ldo) = sum over s < splits of part[s * M * N + m * N + n]
// (+ bias[n]) (+ out[m, n] if accumulate). A block takes 64 consecutive
// elements; its four waves take every fourth split each (four independent
// partial sums per thread) and combine through LDS, in a fixed order.
__global__ __launch_bounds__(kThreads) void msda_split_reduce_kernel(const float* part, int splits,
                                                                     int M, int N, float* out,
                                                                     int64_t ldo, const float* bias,
                                                                     int accumulate) {
    __shared__ float red[4][64];
    const int64_t MN = (int64_t)M * N;
    const int c = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 64 + c;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    if (e < MN) {
        int s = j;
        for (; s + 12 < splits; s += 16) {
            a0 += part[(int64_t)s * MN + e];
            a1 += part[(int64_t)(s + 4) * MN + e];
            a2 += part[(int64_t)(s + 8) * MN + e];
            a3 += part[(int64_t)(s + 12) * MN + e];
        }
        for (; s < splits; s += 4) a0 += part[(int64_t)s * MN + e];
    }
    red[j][c] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    if (j != 0 || e >= MN) return;
    float v = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    const int m = (int)(e / N), n = (int)(e - (int64_t)m * N);
    if (bias) v += bias[n];
    float* dst = out + (int64_t)m * ldo + n;
    if (accumulate) v += *dst;
    *dst = v;
}

// part[s * N + n] = sum of g[r * ldg + n] over the rows of chunk s
// ([s * rows_per, min(R, (s + 1) * rows_per))): 64 columns per block, its four
// waves taking every fourth row, combined through LDS.
__global__ __launch_bounds__(kThreads) void msda_colsum_kernel(const float* g, int64_t ldg, int R,
                                                               int N, int rows_per, float* part) {
    __shared__ float red[4][64];
    const int s = blockIdx.y;
    const int c = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int n = blockIdx.x * 64 + c;
    const int r0 = s * rows_per, r1 = min(R, r0 + rows_per);
    float a0 = 0.0f, a1 = 0.0f;
    if (n < N) {
        int r = r0 + j;
        for (; r + 4 < r1; r += 8) {
            a0 += g[(int64_t)r * ldg + n];
            a1 += g[(int64_t)(r + 4) * ldg + n];
        }
        for (; r < r1; r += 4) a0 += g[(int64_t)r * ldg + n];
    }
    red[j][c] = a0 + a1;
    __syncthreads();
    if (j == 0 && n < N) part[(int64_t)s * N + n] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int splits_for(int64_t R, int64_t in_features, int64_t out_features) {
    // the weight gradient's 128 x 128 tiles times the splits fill the GPU's
    // resident blocks once (kGemmResidentBlocks), at least 256 rows a split
    const int64_t tiles = ((in_features + kTile - 1) / kTile) * ((out_features + kTile - 1) / kTile);
    const int64_t want = std::min<int64_t>((R + 255) / 256, kGemmResidentBlocks / std::max<int64_t>(tiles, 1));
    return (int)std::max<int64_t>(1, std::min<int64_t>(kSplitMax, want));
}

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

}  // namespace

// Shared with the layer entry points (msda_layer.hip): C = A B (+ bias) (+ C)
// as described at GemmArgs; a_kmajor / b_kmajor pick the operand strides.
// With splits > 1 the reduction is split over blocks into `partials`
// (splits * M * N floats) and summed by a second kernel.
namespace {
msda_status_t launch_reduce(const float* part, int splits, int M, int N, float* out, int64_t ldo,
                            const float* bias, bool accumulate, hipStream_t stream) {
    const int64_t n = (int64_t)M * N;
    int acc = accumulate ? 1 : 0;
    void* rargs[] = {&part, &splits, &M, &N, &out, &ldo, &bias, &acc};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&msda_split_reduce_kernel),
                                         dim3((unsigned)((n + 63) / 64)), dim3(kThreads), rargs, 0,
                                         stream);
    return e == hipSuccess ? MSDA_SUCCESS : MSDA_ERROR_LAUNCH;
}
}  // namespace

namespace {

bool operand_vec(const float* P, int64_t ld, bool kmajor, int rows, int K) {
    return aligned(P, 16) && ld % 4 == 0 && (kmajor ? K % 4 == 0 : rows % 4 == 0);
}

}  // namespace

msda_status_t msda_gemm_batch(const GemmSpec* specs, int count, hipStream_t stream) {
    if (count < 1 || count > kMaxGroup) return MSDA_ERROR_INVALID_VALUE;
    GemmGroup grp = {};
    int src[kMaxGroup];   // the spec each launched problem came from
    int n = 0;
    int64_t units = 0;
    bool vec = true;
    for (int i = 0; i < count; ++i) {
        const GemmSpec& sp = specs[i];
        if (sp.a_kmajor != specs[0].a_kmajor || sp.b_kmajor != specs[0].b_kmajor)
            return MSDA_ERROR_INVALID_VALUE;
        if (sp.K2 > 0 && (sp.K % kBK != 0 || sp.splits > 1)) return MSDA_ERROR_INVALID_VALUE;
        if (sp.M == 0 || sp.N == 0) continue;
        src[n] = i;
        GemmArgs& g = grp.g[n++];
        g.A = sp.A;
        g.B = sp.B;
        g.bias = sp.bias;
        g.lda = sp.lda;
        g.ldb = sp.ldb;
        g.M = sp.M;
        g.N = sp.N;
        g.K = sp.K;
        g.A2 = sp.A2;
        g.B2 = sp.B2;
        g.lda2 = sp.lda2;
        g.ldb2 = sp.ldb2;
        g.K2 = sp.K2 > 0 ? sp.K2 : 0;
        const int ktot = g.K + g.K2;
        int splits = std::max(1, sp.splits);
        g.k_split = (int)round_up((ktot + splits - 1) / splits, kBK);
        if (g.k_split == 0) g.k_split = kBK;
        splits = (int)std::max<int64_t>(1, (ktot + g.k_split - 1) / g.k_split);
        g.splits = splits;
        if (splits > 1) {
            g.C = sp.partials;
            g.ldc = sp.N;
            g.bias = nullptr;
            g.accumulate = 0;
            g.split_stride = (int64_t)sp.M * sp.N;
            g.asum = sp.a_colsum ? sp.a_colsum_partials : nullptr;
        } else {
            g.C = sp.C;
            g.ldc = sp.ldc;
            g.accumulate = sp.accumulate ? 1 : 0;
            g.split_stride = 0;
            g.asum = sp.a_colsum;
        }
        g.unit_begin = (int)units;
        units += (int64_t)((sp.M + kTile - 1) / kTile) * ((sp.N + kTile - 1) / kTile) * splits;
        // vector loads: every operand's contiguous dimension a multiple of 4
        // floats, strides too, 16-byte aligned bases
        vec = vec && operand_vec(sp.A, sp.lda, sp.a_kmajor, sp.M, sp.K) &&
              operand_vec(sp.B, sp.ldb, sp.b_kmajor, sp.N, sp.K);
        if (g.K2 > 0)
            vec = vec && operand_vec(sp.A2, sp.lda2, sp.a_kmajor, sp.M, sp.K2) &&
                  operand_vec(sp.B2, sp.ldb2, sp.b_kmajor, sp.N, sp.K2);
    }
    if (n == 0) return MSDA_SUCCESS;
    grp.count = n;
    const bool ak = specs[0].a_kmajor, bk = specs[0].b_kmajor;
    const void* kern = nullptr;
#define MSDA_PICK(AK, BKM)                                                                   \
    if (ak == AK && bk == BKM)                                                               \
        kern = vec ? reinterpret_cast<const void*>(&msda_gemm_kernel<AK, BKM, true>)         \
                   : reinterpret_cast<const void*>(&msda_gemm_kernel<AK, BKM, false>);
    MSDA_PICK(true, true)
    MSDA_PICK(true, false)
    MSDA_PICK(false, true)
    MSDA_PICK(false, false)
#undef MSDA_PICK
    void* args[] = {&grp};
    const hipError_t e =
        hipLaunchKernel(kern, dim3((unsigned)units), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return MSDA_ERROR_LAUNCH;
    for (int i = 0; i < n; ++i) {
        const GemmArgs& g = grp.g[i];
        if (g.splits <= 1) continue;
        const GemmSpec* sp = &specs[src[i]];
        msda_status_t st = launch_reduce(g.C, g.splits, g.M, g.N, sp->C, sp->ldc, sp->bias,
                                         sp->accumulate, stream);
        if (st != MSDA_SUCCESS) return st;
        if (sp->a_colsum) {
            st = launch_reduce(sp->a_colsum_partials, g.splits, 1, g.M, sp->a_colsum, g.M, nullptr,
                               false, stream);
            if (st != MSDA_SUCCESS) return st;
        }
    }
    return MSDA_SUCCESS;
}

msda_status_t msda_gemm(bool a_kmajor, bool b_kmajor, int M, int N, int K, const float* A,
                        int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                        const float* bias, bool accumulate, int splits, float* partials,
                        hipStream_t stream, float* a_colsum, float* a_colsum_partials) {
    GemmSpec sp;
    sp.a_kmajor = a_kmajor;
    sp.b_kmajor = b_kmajor;
    sp.M = M;
    sp.N = N;
    sp.K = K;
    sp.A = A;
    sp.lda = lda;
    sp.B = B;
    sp.ldb = ldb;
    sp.C = C;
    sp.ldc = ldc;
    sp.bias = bias;
    sp.accumulate = accumulate;
    sp.splits = splits;
    sp.partials = partials;
    sp.a_colsum = a_colsum;
    sp.a_colsum_partials = a_colsum_partials;
    return msda_gemm_batch(&sp, 1, stream);
}

// grad_bias[n] = sum over rows of g[r * ldg + n], through `partials`
// (splits * N floats).
msda_status_t msda_colsum(int R, int N, const float* g, int64_t ldg, float* out, int splits,
                          float* partials, bool accumulate, hipStream_t stream) {
    if (N == 0) return MSDA_SUCCESS;
    splits = std::max(1, std::min(splits, std::max(R, 1)));
    int rows_per = (R + splits - 1) / splits;
    if (rows_per == 0) rows_per = 1;
    void* args[] = {&g, &ldg, &R, &N, &rows_per, &partials};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&msda_colsum_kernel),
                                         dim3((unsigned)((N + 63) / 64), (unsigned)splits),
                                         dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return MSDA_ERROR_LAUNCH;
    return launch_reduce(partials, splits, 1, N, out, N, nullptr, accumulate, stream);
}

// Workspace of a linear backward: the weight gradient's split partials and
// the bias gradient's.
size_t msda_linear_workspace_floats(int64_t rows, int64_t in_features, int64_t out_features) {
    const int s = splits_for(rows, in_features, out_features);
    return (size_t)s * (size_t)in_features * (size_t)out_features + (size_t)s * (size_t)out_features;
}

int msda_linear_splits(int64_t rows, int64_t in_features, int64_t out_features) {
    return splits_for(rows, in_features, out_features);
}

namespace {
constexpr int64_t kMaxDim = (int64_t)1 << 30;

msda_status_t check_linear(int64_t rows, int64_t in_f, int64_t out_f) {
    if (rows < 0 || in_f < 1 || out_f < 1) return MSDA_ERROR_INVALID_VALUE;
    if (rows >= kMaxDim || in_f >= (1 << 20) || out_f >= (1 << 20)) return MSDA_ERROR_NOT_SUPPORTED;
    return MSDA_SUCCESS;
}
}  // namespace

extern "C" {

msda_status_t msda_linear_forward(int64_t rows, int64_t in_features, int64_t out_features,
                                  const float* x, const float* weight, const float* bias, float* y,
                                  hipStream_t stream) {
    const msda_status_t st = check_linear(rows, in_features, out_features);
    if (st != MSDA_SUCCESS) return st;
    if (rows == 0) return MSDA_SUCCESS;
    if (!x || !weight || !y) return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(x, 4) || !aligned(weight, 4) || !aligned(y, 4) || !aligned(bias, 4))
        return MSDA_ERROR_INVALID_VALUE;
    // y[r, o] = sum_i x[r, i] W[o, i]: A = x (i-contiguous), B(i, o) = W[o, i]
    return msda_gemm(true, true, (int)rows, (int)out_features, (int)in_features, x, in_features,
                     weight, in_features, y, out_features, bias, false, 1, nullptr, stream);
}

msda_status_t msda_linear_backward_workspace_size(int64_t rows, int64_t in_features,
                                                  int64_t out_features, size_t* bytes) {
    if (!bytes) return MSDA_ERROR_INVALID_VALUE;
    const msda_status_t st = check_linear(rows, in_features, out_features);
    if (st != MSDA_SUCCESS) return st;
    *bytes = msda_linear_workspace_floats(rows, in_features, out_features) * sizeof(float);
    return MSDA_SUCCESS;
}

msda_status_t msda_linear_backward(int64_t rows, int64_t in_features, int64_t out_features,
                                   const float* x, const float* weight, const float* grad_y,
                                   float* grad_x, float* grad_weight, float* grad_bias,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const msda_status_t st = check_linear(rows, in_features, out_features);
    if (st != MSDA_SUCCESS) return st;
    if (!aligned(x, 4) || !aligned(weight, 4) || !aligned(grad_y, 4) || !aligned(grad_x, 4) ||
        !aligned(grad_weight, 4) || !aligned(grad_bias, 4) || !aligned(workspace, 16))
        return MSDA_ERROR_INVALID_VALUE;
    if (rows > 0 && (!grad_y || (grad_x && !weight) || (grad_weight && !x)))
        return MSDA_ERROR_INVALID_VALUE;
    const bool need_ws = grad_weight || grad_bias;
    if (need_ws) {
        const size_t need =
            msda_linear_workspace_floats(rows, in_features, out_features) * sizeof(float);
        if (!workspace || workspace_bytes < need) return MSDA_ERROR_INVALID_VALUE;
    }
    const int R = (int)rows, I = (int)in_features, O = (int)out_features;
    const int splits = splits_for(rows, in_features, out_features);
    float* part_w = static_cast<float*>(workspace);
    float* part_b = part_w ? part_w + (size_t)splits * I * O : nullptr;
    msda_status_t s = MSDA_SUCCESS;
    if (grad_x && R > 0) {
        // dx[r, i] = sum_o dy[r, o] W[o, i]: A = dy (o-contiguous), B(o, i) = W[o * I + i]
        s = msda_gemm(true, false, R, I, O, grad_y, O, weight, I, grad_x, I, nullptr, false, 1,
                      nullptr, stream);
        if (s != MSDA_SUCCESS) return s;
    }
    if (grad_weight) {
        // dW[o, i] = sum_r dy[r, o] x[r, i]: A(o, r) = dy[r * O + o], B(r, i) = x[r * I + i];
        // grad_bias, the sum of A over r, comes out of the same pass
        s = msda_gemm(false, false, O, I, R, grad_y, O, x, I, grad_weight, I, nullptr, false,
                      R == 0 ? 1 : splits, part_w, stream, grad_bias, part_b);
        return s;
    }
    if (grad_bias) s = msda_colsum(R, O, grad_y, O, grad_bias, splits, part_b, false, stream);
    return s;
}

}  // extern "C"
