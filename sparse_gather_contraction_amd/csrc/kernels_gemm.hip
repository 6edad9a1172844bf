// kernels_gemm.hip — dense bf16 / fp16 products on the gfx950 matrix cores for the backward of the fused
// convolution (the gradients of <gy, y> for y = einsum(W, F x); torch-harmonics
// "disco-kernel-dev" page, "Python dispatch layer": the fused autograd function pairs the fused
// forward with the CSR transpose backward).
//
//   g[b, c k, n]  = sum_o W[o, c k] gy[b, o, n]           (n = ho Wo + wo)
//   dW[o, c k]    = sum_{b, n} gy[b, o, n] out[b, c k, n]  (out = F x)
//
// Both are "NT" products C[m][n] = sum_k A[m][k] B[n][k] whose operands are contiguous along the
// reduction index k: g takes A = W^T (rows c k) and B = gy^T (rows n, made by a transpose
// kernel); dW takes A = gy (rows o) and B = out (rows c k), split over the positions with one
// fp32 partial per split, summed afterwards in a fixed order (no atomics).
//
// Tile: 128 x 128 outputs per workgroup of four waves (64 x 64 each, 2 x 2
// v_mfma_f32_32x32x16_bf16 accumulators).  The reduction walks 32-wide chunks; both operand
// chunks (128 rows x 64 bytes) stream into LDS by direct global->LDS loads through a ring of
// three buffers, issued two chunks ahead (the products are short per chunk, so the loads need
// that lead to cover the memory latency).
// A row's four 16-byte column groups are stored XOR-swizzled by (row / 4) % 4 so that the
// 16-byte operand reads of 16 consecutive rows hit distinct LDS banks.
// Workgroups go round the eight XCDs (each with its own L2) by workgroup index; the grid is
// renumbered so that each XCD takes one contiguous run of tiles in the order (split, column tile,
// row tile), and the tiles that share an operand run back to back on one L2.
#include "common.hpp"
#include "kernels.hpp"

namespace disco {

namespace {

constexpr int kGK = 32;      // reduction chunk (elements): 64 bytes per operand row
constexpr int kGRing = 3;    // chunks in flight + the one being multiplied

// Tile shapes: TM x TN outputs per workgroup of WM x WN waves, each wave (TM / WM) x (TN / WN).
//   small: 128 x 128, 2 x 2 waves (64 x 64 each)
//   large: 256 x 256, 2 x 4 waves (128 x 64 each): half the operand bytes per MFMA
template <int TM_, int TN_, int WM_, int WN_>
struct GTile {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int FM = TM / WM / 32, FN = TN / WN / 32;  // 32 x 32 accumulators per wave
    static constexpr int kABytes = TM * kGK * 2, kBBytes = TN * kGK * 2;
    static constexpr int kStage = kABytes + kBBytes;
};
typedef GTile<128, 128, 2, 2> GSmall;
typedef GTile<256, 256, 2, 4> GLarge;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One 32 x 32 x 16 product on the data type's matrix cores (operands travel as raw 16-bit patterns).
template <bool F16>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> the data type's 16-bit pattern, round to nearest even
template <bool F16>
__device__ __forceinline__ bf16_t to16(float v)
{
    if constexpr (F16)
        return __builtin_bit_cast(bf16_t, (_Float16)v);
    else
        return f32_to_bf16(v);
}
typedef void __attribute__((address_space(3))) *lptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Lane i of the instruction writes LDS base `l` + 16 i (buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *l)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l, 16, voff, 0, 0, 0);
}

constexpr uint32_t kOob = 0x80000000u;  // beyond every buffer used here: the load returns zeros

// One operand chunk: rows row0 .. row0+ROWS-1 (valid below nrows), reduction indices k .. k+31
// (valid below k_end; k and k_end are multiples of 8).  LDS slot u (16 bytes) holds row u / 4,
// column group (u % 4) ^ ((row / 4) % 4).  Every thread issues ROWS * 4 / THREADS loads.
template <int ROWS, int THREADS>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t r, int64_t ld, int row0, int nrows, int k, int k_end,
                                           unsigned char *dst, int tid, int wave)
{
    static_assert(ROWS * 4 % THREADS == 0, "whole loads per thread");
#pragma unroll
    for (int i = 0; i < ROWS * 4 / THREADS; ++i) {
        const int u = i * THREADS + tid;
        const int row = u >> 2;
        const int cg = (u & 3) ^ ((row >> 2) & 3);
        const int grow = row0 + row, kk = k + 8 * cg;
        const uint32_t voff = (grow < nrows && kk < k_end) ? (uint32_t)((grow * ld + kk) * 2) : kOob;
        dma16(r, voff, dst + 16 * (i * THREADS + wave * 64));
    }
}

// 16-byte operand of MFMA row `row` (tile-local) for reduction step ks (0 or 1) and lane half h.
__device__ __forceinline__ bf16x8 frag(const unsigned char *op, int row, int ks, int h)
{
    const int slot = (2 * ks + h) ^ ((row >> 2) & 3);
    return *reinterpret_cast<const bf16x8 *>(op + row * 64 + 16 * slot);
}

// C[m][n] = sum_{k in [k_begin, k_end)} A[m][k] B[n][k]; the tile index selects the k range (split).
// OUT_F32: fp32 partial [z][M][N]; else 16-bit C with row stride ldc.  F16: fp16 operands and
// output (else bf16); the operands move as raw 16-bit patterns either way.
template <typename T, bool OUT_F32, bool F16>
__global__ __launch_bounds__(T::kThreads) void gemm_nt_kernel(const bf16_t *__restrict__ A, int64_t lda, int M,
                                                              uint32_t a_bytes, const bf16_t *__restrict__ Bm,
                                                              int64_t ldb, int N, uint32_t b_bytes, int Kd,
                                                              int k_per_split, void *__restrict__ Cout, int64_t ldc,
                                                              int nt_m, int nt_n, int total)
{
    constexpr int FM = T::FM, FN = T::FN;
    constexpr int LOADS = (T::TM + T::TN) * 4 / T::kThreads;  // direct loads per thread per chunk
    __shared__ __attribute__((aligned(16))) unsigned char smem[kGRing * T::kStage];
    const int per_xcd = (int)(gridDim.x >> 3);
    const int L = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (L >= total) return;
    const int tm = L % nt_m, tn = (L / nt_m) % nt_n, z = L / (nt_m * nt_n);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % T::WM, wn = wave / T::WM;
    const int m0 = tm * T::TM, n0 = tn * T::TN;
    const int k_begin = z * k_per_split;
    const int k_end = min(Kd, k_begin + k_per_split);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, a_bytes), rb = make_rsrc(Bm, b_bytes);

    f32x16 d[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int a = 0; a < 16; ++a) d[i][j][a] = 0.0f;

    const int nk = k_end > k_begin ? (k_end - k_begin + kGK - 1) / kGK : 0;
    // chunk t lives in ring slot t % 3
    auto issue = [&](int t) {
        unsigned char *dst = smem + (t % kGRing) * T::kStage;
        const int k = k_begin + t * kGK;
        load_chunk<T::TM, T::kThreads>(ra, lda, m0, M, k, k_end, dst, tid, wave);
        load_chunk<T::TN, T::kThreads>(rb, ldb, n0, N, k, k_end, dst + T::kABytes, tid, wave);
    };
    if (nk > 0) issue(0);
    if (nk > 1) issue(1);
    const int r = lane & 31, h = lane >> 5;
    for (int t = 0; t < nk; ++t) {
        // this thread's loads of chunk t have landed (those of chunk t + 1 may still be in flight)
        static_assert(LOADS == 4, "the wait below leaves one chunk of four loads in flight");
        if (t + 1 < nk)
            __builtin_amdgcn_s_waitcnt(0x074);  // vmcnt <= 4, lgkmcnt 0
        else
            __builtin_amdgcn_s_waitcnt(0);
        // A bare barrier: __syncthreads() adds a workgroup release fence, which the compiler turns
        // into a wait for every direct load into LDS in flight, chunk t + 1's too.  The wait above
        // covers this thread's loads of chunk t; the compiler-level fences keep LDS accesses on
        // their side of the barrier.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // everyone's have landed; every wave is done with chunk t - 1, whose slot is refilled
        asm volatile("" ::: "memory");
        if (t + 2 < nk) issue(t + 2);
        const unsigned char *cur = smem + (t % kGRing) * T::kStage;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = frag(cur, (T::TM / T::WM) * wm + 32 * i + r, ks, h);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = frag(cur + T::kABytes, (T::TN / T::WN) * wn + 32 * j + r, ks, h);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    d[i][j] = mma<F16>(fa[i], fb[j], d[i][j]);
        }
    }

    // lane (column r, half h) holds rows 8 (a / 4) + 4 h + a % 4 of each 32 x 32 accumulator
    if constexpr (!OUT_F32) {
        // bf16 output through LDS (the ring is free: the last chunk waited for every load): pass p
        // stages the TM / WM rows of the waves with wm == p as [row][TN + 8] bf16 (the 16-byte pad
        // puts rows 4 apart, the two lane halves, on different banks), then every thread writes
        // 16-byte row segments instead of 2-byte elements.
        constexpr int PR = T::TM / T::WM, PITCH = T::TN + 8;
        static_assert(PR * PITCH * 2 <= kGRing * T::kStage, "a pass fits the ring's space");
        bf16_t *tile = reinterpret_cast<bf16_t *>(smem);
        const bool vec = ldc % 8 == 0 && ((uintptr_t)Cout % 16) == 0;
#pragma unroll
        for (int pass = 0; pass < T::WM; ++pass) {
            __syncthreads();  // every wave is done with the ring, or with the previous pass's tile
            if (wm == pass) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int a = 0; a < 16; ++a) {
                            const int ml = 32 * i + 8 * (a >> 2) + 4 * h + (a & 3);
                            tile[ml * PITCH + (T::TN / T::WN) * wn + 32 * j + r] = to16<F16>(d[i][j][a]);
                        }
            }
            __syncthreads();
            for (int u = tid; u < PR * (T::TN / 8); u += T::kThreads) {
                const int ml = u / (T::TN / 8), seg = u - ml * (T::TN / 8);
                const int m = m0 + PR * pass + ml, n = n0 + 8 * seg;
                if (m >= M || n >= N) continue;
                bf16_t *dst = reinterpret_cast<bf16_t *>(Cout) + (int64_t)m * ldc + n;
                const bf16_t *src = tile + ml * PITCH + 8 * seg;
                if (vec && n + 8 <= N) {
                    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
                } else {
                    for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = src[e];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + (T::TN / T::WN) * wn + 32 * j + r;
            if (n >= N) continue;
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int m = m0 + (T::TM / T::WM) * wm + 32 * i + 8 * (a >> 2) + 4 * h + (a & 3);
                if (m >= M) continue;
                if constexpr (OUT_F32)
                    reinterpret_cast<float *>(Cout)[((int64_t)z * M + m) * N + n] = d[i][j][a];
                else
                    reinterpret_cast<bf16_t *>(Cout)[(int64_t)m * ldc + n] = to16<F16>(d[i][j][a]);
            }
        }
}

// dst[c][r] = src[r][c] for an R x Cn bf16 matrix (row strides Cn and R); 64 x 64 tiles via LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const bf16_t *__restrict__ src, bf16_t *__restrict__ dst,
                                                        int R, int Cn)
{
    __shared__ bf16_t t[64][66];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int rr = i >> 6, cc = i & 63;
        const int gr = r0 + rr, gc = c0 + cc;
        t[rr][cc] = (gr < R && gc < Cn) ? src[(int64_t)gr * Cn + gc] : (bf16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int cc = i >> 6, rr = i & 63;
        const int gr = r0 + rr, gc = c0 + cc;
        if (gr < R && gc < Cn) dst[(int64_t)gc * R + gr] = t[rr][cc];
    }
}

// dW[o][col0 + m] = 16-bit(sum_{z < Z} P[z][o][m]) in increasing z.
template <bool F16>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ P, int Z, int Co, int Mc,
                                                              bf16_t *__restrict__ dW, int64_t ldw, int col0)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)Co * Mc) return;
    const int o = (int)(i / Mc), m = (int)(i % Mc);
    float acc = 0.0f;
    for (int z = 0; z < Z; ++z) acc += P[((int64_t)z * Co + o) * Mc + m];
    dW[(int64_t)o * ldw + col0 + m] = to16<F16>(acc);
}

template <typename T, bool F16>
hipError_t launch_gemm_tiles(const GemmNtLaunch &g, hipStream_t stream)
{
    const int splits = (g.out_f32 && g.k_per_split > 0) ? (g.Kd + g.k_per_split - 1) / g.k_per_split : 1;
    const int kps = g.k_per_split > 0 ? g.k_per_split : g.Kd;
    const int nt_m = (g.M + T::TM - 1) / T::TM, nt_n = (g.N + T::TN - 1) / T::TN;
    const int64_t total = (int64_t)nt_m * nt_n * splits;
    if (total >= ((int64_t)1 << 31) - 8) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 7) / 8 * 8));  // a multiple of the eight XCDs
    if (g.out_f32)
        hipLaunchKernelGGL((gemm_nt_kernel<T, true, F16>), grid, dim3(T::kThreads), 0, stream, (const bf16_t *)g.A, g.lda,
                           g.M, g.a_bytes, (const bf16_t *)g.B, g.ldb, g.N, g.b_bytes, g.Kd, kps, g.C, g.ldc, nt_m,
                           nt_n, (int)total);
    else
        hipLaunchKernelGGL((gemm_nt_kernel<T, false, F16>), grid, dim3(T::kThreads), 0, stream, (const bf16_t *)g.A, g.lda,
                           g.M, g.a_bytes, (const bf16_t *)g.B, g.ldb, g.N, g.b_bytes, g.Kd, kps, g.C, g.ldc, nt_m,
                           nt_n, (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNtLaunch &g, hipStream_t stream)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    // the large tile when both output dimensions fill it
    const bool large = g.M >= 256 && g.N >= 256;
    if (g.f16) return large ? launch_gemm_tiles<GLarge, true>(g, stream) : launch_gemm_tiles<GSmall, true>(g, stream);
    return large ? launch_gemm_tiles<GLarge, false>(g, stream) : launch_gemm_tiles<GSmall, false>(g, stream);
}

namespace {

// one thread per element of W' (C, Co, 16)
__global__ __launch_bounds__(256) void permute_w16_kernel(const bf16_t *__restrict__ W, bf16_t *__restrict__ Wt, int Co,
                                                         int C, int K)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)C * Co * 16) return;
    const int k = (int)(i & 15);
    const int64_t co = i >> 4;
    const int o = (int)(co % Co), c = (int)(co / Co);
    Wt[i] = k < K ? W[((int64_t)o * C + c) * K + k] : (bf16_t)0;
}

}  // namespace

hipError_t launch_permute_w16(const void *W, void *Wt, int Co, int C, int K, hipStream_t stream)
{
    const int64_t n = (int64_t)C * Co * 16;
    if (n == 0) return hipSuccess;
    if (K < 1 || K > 16 || (n + 255) / 256 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(permute_w16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, (const bf16_t *)W,
                       (bf16_t *)Wt, Co, C, K);
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void *src, void *dst, int R, int Cn, hipStream_t stream)
{
    if (R <= 0 || Cn <= 0) return hipSuccess;
    dim3 grid((Cn + 63) / 64, (R + 63) / 64);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, (const bf16_t *)src, (bf16_t *)dst, R, Cn);
    return hipGetLastError();
}

hipError_t launch_reduce_partials(const float *P, int Z, int Co, int Mc, void *dW, int64_t ldw, int col0, bool f16,
                                  hipStream_t stream)
{
    const int64_t n = (int64_t)Co * Mc;
    if (n <= 0) return hipSuccess;
    if (f16)
        hipLaunchKernelGGL(reduce_partials_kernel<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, P, Z,
                           Co, Mc, (bf16_t *)dW, ldw, col0);
    else
        hipLaunchKernelGGL(reduce_partials_kernel<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, P, Z,
                           Co, Mc, (bf16_t *)dW, ldw, col0);
    return hipGetLastError();
}


}  // namespace disco
