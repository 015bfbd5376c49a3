// Kernels of the BRA module around the method (gfx950): the per-token linear
// maps that make Q, K, V from x and the optional output projection, and the
// float64 projection of x's region means that routing uses.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3: q_proj / k_proj / v_proj of x, region means of q and k), p2 =
// snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的计算
// 范式" (§2: region means over the region axes).
//
// Routing needs the region means of Q = x Wq^T + bq and K.  A region mean is
// a weighted sum with weights summing to one, so it commutes with the
// per-token linear map: mean(Q) = mean(x) Wq^T + bq.  The module therefore
// pools x once (float64, exact for bf16 inputs) and projects the means in
// float64 -- the routing sees the same means as a float64 evaluation of the
// definition, not means of the rounded Q and K.

#include "device_common.h"

namespace bra {
namespace {

constexpr int kLinRows = 128;     // tokens per workgroup (32 per wavefront)
constexpr int kLinCols = 64;      // output features per workgroup
constexpr int kLinKChunk = 256;   // weight columns staged in LDS at a time
constexpr uint32_t kLinOob = 0x80000000u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lin_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct LinArgs {
  const void* x;        // [T, K]
  const void* w;        // [N, K]
  const float* b;       // [N] or null
  void* y[3];           // output groups: columns [g*ng, (g+1)*ng) go to y[g], [T, ng]
  int ng;               // columns per output group
  int T, K, N;
  int col_tiles, tiles, per_xcd;
};

// Y = X W^T + b on the matrix cores, computed as Y^T = W X^T so that a lane
// ends with 4 consecutive output features of one token (one 8- or 16-byte
// store).  A workgroup owns 128 tokens x 64 features; wavefront w its tokens
// 32w .. 32w+31 (two 16-token blocks) against all 64 features (four 16-row
// blocks of W).  W's 64 x 256 chunk is staged in LDS with its 16-byte chunks
// XOR-swizzled by row; X is read straight from memory in the operand layout
// (one 16-byte row segment per lane).  Tiles go to XCDs in contiguous
// ranges, features fastest, so the workgroups that share X rows share an L2.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void linear_kernel(LinArgs a) {
  constexpr int ES = BF16 ? 2 : 4;                 // element bytes
  constexpr int KSTEP = BF16 ? 32 : 4;             // k per MFMA
  constexpr int CE = 16 / ES;                      // elements per 16-byte chunk
  extern __shared__ __align__(16) unsigned char lds[];
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int id = xcd * a.per_xcd + loc;
  if (loc >= a.per_xcd || id >= a.tiles) return;   // uniform; no barrier passed yet
  const int rt = id / a.col_tiles, ct = id - rt * a.col_tiles;
  const int t0 = rt * kLinRows, n0 = ct * kLinCols;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const auto X = lin_rsrc(a.x, (uint32_t)a.T * a.K * ES);
  const unsigned char* W = (const unsigned char*)a.w;

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < a.K; kc += kLinKChunk) {
    const int kn = min(kLinKChunk, a.K - kc);      // a multiple of 32
    const int cpr = kn / CE;                        // 16-byte chunks per staged row
    const int sw = cpr % 8 == 0 ? 7 : 3;            // cpr is a multiple of 4
    if (kc > 0) __syncthreads();                   // previous chunk fully read
    // stage W[n0 .. n0+63][kc .. kc+kn): row r, chunk c at chunk c ^ (r & sw)
    for (int e = tid; e < kLinCols * cpr; e += kThreads) {
      const int r = e / cpr, c = e - r * cpr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n0 + r < a.N)
        v = *(const uint4*)(W + ((size_t)(n0 + r) * a.K + kc + c * CE) * ES);
      *(uint4*)(lds + (r * cpr + (c ^ (r & sw))) * 16) = v;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; kk += KSTEP) {
      // X^T operand: token 16tb + lq of this wavefront, k = kc + kk + (8 | 1) lg
      if constexpr (BF16) {
        bf16x8 xb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = t0 + 32 * wave + 16 * tb + lq;
          const uint32_t off = t < a.T ? ((uint32_t)t * a.K + kc + kk + 8 * lg) * 2 : kLinOob;
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(X, off, 0, 0);
          xb[tb] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int r = 16 * nb + lq;
          const int c = (kk >> 3) + lg;            // chunk of k = kk + 8 lg
          const bf16x8 wa = *(const bf16x8*)(lds + (r * cpr + (c ^ (r & sw))) * 16);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            acc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb[tb], acc[tb][nb], 0, 0, 0);
        }
      } else {
        float xf[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = t0 + 32 * wave + 16 * tb + lq;
          const uint32_t off = t < a.T ? ((uint32_t)t * a.K + kc + kk + lg) * 4 : kLinOob;
          xf[tb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(X, off, 0, 0));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int r = 16 * nb + lq;
          const int k = kk + lg, c = k >> 2;
          const float wa = *(const float*)(lds + (r * cpr + (c ^ (r & sw))) * 16 + (k & 3) * 4);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            acc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa, xf[tb], acc[tb][nb], 0, 0, 0);
        }
      }
    }
  }

  // lane (lq, lg) holds Y[token 16tb + lq][features 16nb + 4lg + 0..3]
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 16 * nb + 4 * lg;
    const bool nok = n < a.N;                      // N % 4 == 0: all four or none
    const int g = nok ? n / a.ng : 0, col = n - g * a.ng;
    float bb[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.b && nok) {
      const float4 bv = *(const float4*)(a.b + n);
      bb[0] = bv.x; bb[1] = bv.y; bb[2] = bv.z; bb[3] = bv.w;
    }
    const auto Y = lin_rsrc(a.y[g], (uint32_t)a.T * a.ng * ES);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = t0 + 32 * wave + 16 * tb + lq;
      const uint32_t off =
          (nok && t < a.T) ? ((uint32_t)t * a.ng + col) * ES : kLinOob;
      const f32x4 v = acc[tb][nb];
      if constexpr (BF16) {
        const u32x2 p = {pack_bf16x2(v[0] + bb[0], v[1] + bb[1]),
                         pack_bf16x2(v[2] + bb[2], v[3] + bb[3])};
        __builtin_amdgcn_raw_buffer_store_b64(p, Y, off, 0, 0);
      } else {
        const u32x4 p = {__float_as_uint(v[0] + bb[0]), __float_as_uint(v[1] + bb[1]),
                         __float_as_uint(v[2] + bb[2]), __float_as_uint(v[3] + bb[3])};
        __builtin_amdgcn_raw_buffer_store_b128(p, Y, off, 0, 0);
      }
    }
  }
}

// qm = xm Wq^T + bq and km = xm Wk^T + bk in float64 (Wq, Wk: rows 0..C-1
// and C..2C-1 of w_qkv), one 16 x 16 output tile per wavefront on
// v_mfma_f64_16x16x4f64.  Each lane feeds 4 consecutive channels as the k
// slots of 4 successive MFMAs (the same permutation on both operands).
struct MeansArgs {
  const double* xm;     // [rows, C]
  const void* w;        // w_qkv [3C, C]
  const float* b;       // b_qkv [3C] or null
  double* qm;           // [rows, C]
  double* km;           // [rows, C]
  int rows, C;
  int col_tiles, tiles;
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void means_proj_kernel(MeansArgs a) {
  const int tile = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (tile >= a.tiles) return;                    // no barrier in this kernel
  const int lane = threadIdx.x & 63, l16 = lane & 15, lk = lane >> 4;
  const int rt = tile / a.col_tiles, ct = tile - rt * a.col_tiles;
  const int r0 = rt * 16, n0 = ct * 16;           // n over the 2C columns (q then k)
  const int C = a.C;
  const double* xp = a.xm + (size_t)min(r0 + l16, a.rows - 1) * C + 4 * lk;
  const int wn = n0 + l16;                         // weight row (< 2C: C % 16 == 0)
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  for (int c = 0; c < C; c += 16) {
    const double4 xa = *(const double4*)(xp + c);
    double wb[4];
    if constexpr (BF16) {
      const uint2 u = *(const uint2*)((const uint16_t*)a.w + (size_t)wn * C + c + 4 * lk);
      wb[0] = bf16_lo(u.x); wb[1] = bf16_hi(u.x); wb[2] = bf16_lo(u.y); wb[3] = bf16_hi(u.y);
    } else {
      const float4 u = *(const float4*)((const float*)a.w + (size_t)wn * C + c + 4 * lk);
      wb[0] = u.x; wb[1] = u.y; wb[2] = u.z; wb[3] = u.w;
    }
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.x, wb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.y, wb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.z, wb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa.w, wb[3], acc, 0, 0, 0);
  }
  // D layout (f64 16x16x4): lane holds column l16 of the tile, rows lk + 4i
  const int n = n0 + l16;
  const double bias = a.b ? (double)a.b[n] : 0.0;
  double* dst = n < C ? a.qm : a.km;
  const int col = n < C ? n : n - C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + lk + 4 * i;
    if (r < a.rows) dst[(size_t)r * C + col] = acc[i] + bias;
  }
}

}  // namespace

hipError_t launch_linear(const void* x, int T, int K, const void* w, const float* b, int N,
                         void* const* y, int groups, bool bf16, hipStream_t st) {
  if (T <= 0 || K <= 0 || N <= 0 || K % 32 || N % 4 || groups < 1 || groups > 3 ||
      N % groups || (N / groups) % 4)
    return hipErrorInvalidValue;
  const int es = bf16 ? 2 : 4;
  // buffer offsets are 32-bit: every operand below 2 GiB
  if ((long long)T * K * es >= (long long)kLinOob || (long long)T * (N / groups) * es >= (long long)kLinOob)
    return hipErrorNotSupported;
  LinArgs a;
  a.x = x; a.w = w; a.b = b;
  for (int g = 0; g < 3; ++g) a.y[g] = g < groups ? y[g] : y[0];
  a.ng = N / groups;
  a.T = T; a.K = K; a.N = N;
  a.col_tiles = (N + kLinCols - 1) / kLinCols;
  a.tiles = ((T + kLinRows - 1) / kLinRows) * a.col_tiles;
  a.per_xcd = (a.tiles + kXcds - 1) / kXcds;
  const size_t lds = (size_t)kLinCols * (K < kLinKChunk ? K : kLinKChunk) * es;
  const dim3 grid((unsigned)(a.per_xcd * kXcds));
  if (bf16)
    hipLaunchKernelGGL(linear_kernel<true>, grid, dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL(linear_kernel<false>, grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_means_proj(const double* xm, int rows, int C, const void* w_qkv,
                             const float* b_qkv, bool bf16, double* qm, double* km,
                             hipStream_t st) {
  if (rows <= 0 || C <= 0 || C % 16) return hipErrorInvalidValue;
  MeansArgs a;
  a.xm = xm; a.w = w_qkv; a.b = b_qkv; a.qm = qm; a.km = km;
  a.rows = rows; a.C = C;
  a.col_tiles = 2 * C / 16;
  a.tiles = ((rows + 15) / 16) * a.col_tiles;
  const dim3 grid((unsigned)((a.tiles + kWaves - 1) / kWaves));
  if (bf16)
    hipLaunchKernelGGL(means_proj_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(means_proj_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace bra
