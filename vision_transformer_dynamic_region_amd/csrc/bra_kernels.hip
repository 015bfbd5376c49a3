// HIP kernels for the Bi-Level Routing Attention forward pass on gfx950.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析",
// p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的
// 计算范式", p5 = hyper.ai abstract of arXiv 2303.08810.
//
// Layouts: Q, K, V, out are [B, H, W, C] channels-last.  A region r = (ry, rx)
// of the S x S grid covers rows ry*hs .. ry*hs+hs-1 and columns
// rx*ws .. rx*ws+ws-1; its pixel t (row-major inside the region) sits at
// (ry*hs + t / ws, rx*ws + t % ws)  (p1 §3 partition).  Nothing is copied
// into a region layout: every kernel computes these addresses directly.

#include <hip/hip_runtime.h>
#include <climits>
#include <type_traits>
#include <stdint.h>

#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 wavefronts of 64
constexpr int kWaves = 4;
constexpr int kXcds = 8;        // MI355X: workgroups go round-robin to 8 XCDs

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Expand 16 bytes of elements into floats.  bf16: 8 values; f32: 4 values.
template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& u, float* f) {
  if constexpr (BF16) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  } else {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
}

__device__ __forceinline__ size_t pixel_offset(int b, int y, int x, const Shape& s) {
  return (((size_t)b * s.H + y) * s.W + x) * (size_t)s.C;
}

// ---------------------------------------------------------------------------
// Pool: region means of Q and K in float64 (p1 §3 region-mean step; p2 §2).
// One workgroup per (image, region).  Each thread owns one 16-byte channel
// group and a strided subset of the region's pixels; partial sums meet in LDS
// and are added in a fixed order, so the result is deterministic.  Summing
// bf16 or f32 values into float64 is exact or within one rounding of the
// exact sum, so the route below sees the same means as an fp64 reference.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void pool_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k,
    double* __restrict__ qm, double* __restrict__ km, Shape s) {
  constexpr int VEC = BF16 ? 8 : 4;
  __shared__ double red[2][kThreads * VEC];
  const int br = blockIdx.x;
  const int b = br / s.R, r = br - b * s.R;
  const int ry = r / s.S, rx = r - ry * s.S;
  const int G = s.C / VEC;               // 16-byte groups per pixel
  const double inv_n = 1.0 / (double)s.n;
  for (int g0 = 0; g0 < G; g0 += kThreads) {
    const int Gc = min(kThreads, G - g0);
    const int P = kThreads / Gc;         // pixel lanes
    const int g = threadIdx.x % Gc, pl = threadIdx.x / Gc;
    double aq[VEC], ak[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) { aq[e] = 0.0; ak[e] = 0.0; }
    if (pl < P) {
      for (int t = pl; t < s.n; t += P) {
        const int ty = t / s.ws, tx = t - ty * s.ws;
        const size_t off = pixel_offset(b, ry * s.hs + ty, rx * s.ws + tx, s) / VEC + g0 + g;
        const uint4 uq = q[off];
        const uint4 uk = k[off];
        float fq[VEC], fk[VEC];
        unpack16<BF16>(uq, fq);
        unpack16<BF16>(uk, fk);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { aq[e] += (double)fq[e]; ak[e] += (double)fk[e]; }
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        red[0][(pl * Gc + g) * VEC + e] = aq[e];
        red[1][(pl * Gc + g) * VEC + e] = ak[e];
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < Gc * VEC; c += kThreads) {
      double sq = 0.0, sk = 0.0;
      for (int p = 0; p < P; ++p) { sq += red[0][p * Gc * VEC + c]; sk += red[1][p * Gc * VEC + c]; }
      const size_t o = (size_t)br * s.C + (size_t)g0 * VEC + c;
      qm[o] = sq * inv_n;
      km[o] = sk * inv_n;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Route: A[r][s] = route_scale * <q_r[r], k_r[s]> in float64, then per row the
// topk largest entries, largest first, equal values by lower index (p1 §3
// affinity and top-k; p2 §4 scaled affinity).  One workgroup per
// (image, block of kRouteRows rows); the rows' q means sit in LDS, the
// affinity rows too; nothing of A is written to memory.
// Values are ranked through an order-preserving int64 key (after turning -0
// into +0 so that 0 and -0 tie, as they compare equal).
// ---------------------------------------------------------------------------
constexpr int kRouteRows = 8;
constexpr int kRouteMaxJ = 16;    // R <= 1024 = 16 candidates per lane

__device__ __forceinline__ long long order_key(double v) {
  v = v + 0.0;                                   // -0 -> +0
  long long k = __double_as_longlong(v);
  return k ^ ((k >> 63) & 0x7fffffffffffffffLL);
}

// true if (ka, ia) ranks before (kb, ib)
__device__ __forceinline__ bool ranks_before(long long ka, int ia, long long kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kThreads) void route_kernel(
    const double* __restrict__ qm, const double* __restrict__ km, Shape s,
    double scale, int32_t* __restrict__ idx, float* __restrict__ logits,
    int use_select) {
  extern __shared__ double rsm[];
  const int R = s.R, C = s.C, topk = s.topk;
  const int nrb = (R + kRouteRows - 1) / kRouteRows;
  const int b = blockIdx.x / nrb, r0 = (blockIdx.x - b * nrb) * kRouteRows;
  const int rows = min(kRouteRows, R - r0);
  double* qs = rsm;                       // [kRouteRows][C]
  double* a = rsm + kRouteRows * C;       // [kRouteRows][R]
  const double* qsrc = qm + ((size_t)b * R + r0) * C;
  for (int i = threadIdx.x; i < rows * C; i += kThreads) qs[i] = qsrc[i];
  __syncthreads();
  const double* kimg = km + (size_t)b * R * C;
  for (int i = threadIdx.x; i < rows * R; i += kThreads) {
    const int rl = i / R, sc = i - rl * R;
    const double* kr = kimg + (size_t)sc * C;
    const double* qr = qs + rl * C;
    double acc = 0.0;
    for (int c = 0; c < C; ++c) acc = fma(qr[c], kr[c], acc);
    a[rl * R + sc] = scale * acc;
  }
  __syncthreads();
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int rl = wave; rl < rows; rl += kWaves) {
    const double* ar = a + rl * R;
    int32_t* irow = idx + ((size_t)b * R + r0 + rl) * topk;
    float* lrow = logits ? logits + ((size_t)b * R + r0 + rl) * topk : nullptr;
    if (!use_select) {
      // rank by counting: rank(s) = #{s' ranking before s}
      for (int sc = lane; sc < R; sc += 64) {
        const double v = ar[sc];
        const long long kv = order_key(v);
        int rank = 0;
        for (int s2 = 0; s2 < R; ++s2) rank += ranks_before(order_key(ar[s2]), s2, kv, sc) ? 1 : 0;
        if (rank < topk) {
          irow[rank] = sc;
          if (lrow) lrow[rank] = (float)v;
        }
      }
    } else {
      // topk rounds of a wavefront-wide arg-max over the remaining entries
      long long keys[kRouteMaxJ];
      const int J = (R + 63) / 64;
#pragma unroll
      for (int j = 0; j < kRouteMaxJ; ++j)
        keys[j] = (j < J && lane + 64 * j < R) ? order_key(ar[lane + 64 * j]) : LLONG_MIN;
      unsigned taken = 0;
      for (int kk = 0; kk < topk; ++kk) {
        long long bk = LLONG_MIN;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kRouteMaxJ; ++j) {
          const int sc = lane + 64 * j;
          if (j < J && sc < R && !((taken >> j) & 1u) && ranks_before(keys[j], sc, bk, bi)) {
            bk = keys[j];
            bi = sc;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const long long ok = __shfl_xor(bk, off);
          const int oi = __shfl_xor(bi, off);
          if (ranks_before(ok, oi, bk, bi)) { bk = ok; bi = oi; }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == 0) {
          irow[kk] = bi;
          if (lrow) lrow[kk] = (float)ar[bi];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 4-channel loads and stores (global memory or LDS) in float.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load4(const void* base, size_t off, float* f) {
  if constexpr (BF16) {
    const uint2 u = *(const uint2*)((const uint16_t*)base + off);
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  } else {
    const float4 u = *(const float4*)((const float*)base + off);
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, size_t off, const float* f) {
  if constexpr (BF16) {
    uint2 u;
    u.x = pack_bf16x2(f[0], f[1]);
    u.y = pack_bf16x2(f[2], f[3]);
    *(uint2*)((uint16_t*)base + off) = u;
  } else {
    *(float4*)((float*)base + off) = make_float4(f[0], f[1], f[2], f[3]);
  }
}

// ---------------------------------------------------------------------------
// LePE arithmetic shared by the fused attention epilogue and the standalone
// kernel (p2 §4 depthwise Conv2d with zero padding ks//2 and one filter per
// channel; p1 §3 adds it to the attention output):
//   L[y,x,c] = bias[c] + sum_{i,j} w[c,i,j] * V[y+i-ks/2, x+j-ks/2, c]
// Both stage a zero-padded tile of V (th + ks - 1 rows by tw + ks - 1
// columns, all channels of a slice) and the weights as [tap][channel] in
// LDS.  A thread then owns 2 channels of one column over kLepeRows output
// rows and walks the kLepeRows + ks - 1 input rows once: every input row
// feeds each output row it touches, so a V element is read ks times per
// strip, not ks*ks times.  Its 2*ks*ks weights stay in registers.
// ---------------------------------------------------------------------------
constexpr int kLepeRows = 8;

template <bool BF16>
__device__ __forceinline__ void load2(const void* base, size_t off, float* f) {
  if constexpr (BF16) {
    const uint32_t u = *(const uint32_t*)((const uint16_t*)base + off);
    f[0] = bf16_lo(u); f[1] = bf16_hi(u);
  } else {
    const float2 u = *(const float2*)((const float*)base + off);
    f[0] = u.x; f[1] = u.y;
  }
}

// Convolve a staged tile.  Hs: [(th+KS-1)*(tw+KS-1)][hc] elements, Wt:
// [KS*KS][hc] floats, bias: global [>= c_base + hc] or null.  Calls
// emit(y, x, c, v0, v1) for the tile's output pixel (y, x) and local
// channels c, c+1.
template <bool BF16, int KS, typename Emit>
__device__ __forceinline__ void conv_tile(const void* Hs, const float* Wt, const float* bias,
                                          int c_base, int th, int tw, int hc, Emit emit) {
  const int hw = tw + KS - 1, hh = th + KS - 1;
  const int G2 = hc / 2;
  const int strips = (th + kLepeRows - 1) / kLepeRows;
  for (int item = threadIdx.x; item < G2 * tw * strips; item += kThreads) {
    const int c = 2 * (item % G2), rest = item / G2;
    const int x = rest % tw, y0 = (rest / tw) * kLepeRows;
    float wr[KS * KS][2];
#pragma unroll
    for (int tap = 0; tap < KS * KS; ++tap) {
      const float2 u = *(const float2*)(Wt + tap * hc + c);
      wr[tap][0] = u.x;
      wr[tap][1] = u.y;
    }
    float acc[kLepeRows][2];
    float b0 = 0.f, b1 = 0.f;
    if (bias) {
      b0 = bias[c_base + c];
      b1 = bias[c_base + c + 1];
    }
#pragma unroll
    for (int r = 0; r < kLepeRows; ++r) {
      acc[r][0] = b0;
      acc[r][1] = b1;
    }
#pragma unroll
    for (int dy = 0; dy < kLepeRows + KS - 1; ++dy) {
      // rows past the tile only feed output rows that are not emitted;
      // clamping keeps their reads inside the staged tile
      const int hy = min(y0 + dy, hh - 1);
      float vv[KS][2];
#pragma unroll
      for (int j = 0; j < KS; ++j) load2<BF16>(Hs, (size_t)(hy * hw + x + j) * hc + c, vv[j]);
      // input row dy feeds output row r = dy - i through kernel row i
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int r = dy - i;
        if (r < 0 || r >= kLepeRows) continue;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          acc[r][0] = fmaf(wr[i * KS + j][0], vv[j][0], acc[r][0]);
          acc[r][1] = fmaf(wr[i * KS + j][1], vv[j][1], acc[r][1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep one input row live at a time
    }
#pragma unroll
    for (int r = 0; r < kLepeRows; ++r)
      if (y0 + r < th) emit(y0 + r, x, c, acc[r][0], acc[r][1]);
  }
}

// Stage the zero-padded V tile whose top-left output pixel is (y0, x0) and
// the weights of channels [c0, c0 + hc) into LDS.
template <bool BF16, int KS>
__device__ __forceinline__ void stage_halo(const void* V, const float* w, int b, int y0, int x0,
                                           int th, int tw, int c0, int hc, const Shape& s,
                                           void* Hs, float* Wt) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int P = KS / 2;
  const int hw = tw + KS - 1, hh = th + KS - 1;
  const int G = hc / VEC;
  for (int e = threadIdx.x; e < hh * hw * G; e += kThreads) {
    const int pix = e / G, g = e - pix * G;
    const int hy = pix / hw, hx = pix - hy * hw;
    const int y = y0 + hy - P, x = x0 + hx - P;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (y >= 0 && y < s.H && x >= 0 && x < s.W)
      val = *(const uint4*)((const T*)V + pixel_offset(b, y, x, s) + c0 + (size_t)g * VEC);
    *(uint4*)((T*)Hs + (size_t)pix * hc + g * VEC) = val;
  }
  for (int e = threadIdx.x; e < KS * KS * hc; e += kThreads) {
    const int c = e / (KS * KS), tap = e - c * (KS * KS);
    Wt[tap * hc + c] = w[(size_t)(c0 + c) * (KS * KS) + tap];
  }
}

// ---------------------------------------------------------------------------
// Gather-attention (p1 §3 gather + softmax attention; p5 token-to-token
// attention over the union of the routed regions), flash style, with the
// LePE term fused into the epilogue.
//
// One workgroup per (image, query region, task group).  A task is one head
// and a block of 16 query pixels; a workgroup owns up to kWaves*kTasksPerWave
// tasks.  The keys of the region -- the tokens of the topk routed regions, in
// route order -- are staged chunk by chunk into LDS straight from their
// NHWC rows (the gathered K/V are never written to memory), all heads at
// once.  Each wavefront then runs its tasks over the chunk in steps of 32
// keys with an online softmax:
//
//   S^T[key][q] = K[key] . Q[q]        MFMA 16x16x32 (bf16) or 8 x 16x16x4 (f32)
//   O^T[d][q]  += V^T[d][key] P^T[key][q]
//
// Computing the transposed products puts one query in each lane column, so
// the softmax statistics and the output rows of a query live in the same
// lanes (lane % 16 = query, lane / 16 = 4-row slice of the MFMA output).
// Per lane the 8 K-dimension elements of every MFMA operand are taken from
// the same (lane / 16, slot) pairs on both sides, so any internal ordering of
// the K dimension by the matrix core gives the same sum.  In bf16 the
// probabilities enter the PV product as a hi + lo pair of bf16 values (two
// MFMAs), so P carries ~16 bits, not 8; Q, K, V are exact bf16 inputs.
//
// Epilogue (KS > 0): the K/V staging area is reused for a zero-padded V halo
// tile of the region (hs+KS-1 by ws+KS-1 pixels), the LePE weights as
// [tap][channel] and an fp32 tile L[pixel][channel]; L is added to the
// normalised attention output before the single rounding to the output type.
// With `accumulate` the kernel instead adds what `out` already holds (the
// LePE term written there by the standalone kernel).
// ---------------------------------------------------------------------------
constexpr int kHeadDim = 32;
constexpr int kTasksPerWave = 2;
constexpr int kTasksPerBlock = kWaves * kTasksPerWave;
constexpr int kStep = 32;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  void* out;
  const float* w;       // fused LePE weights [C, KS, KS] (KS > 0)
  const float* bias;    // fused LePE bias [C] or null
  Shape s;
  float scale_log2;     // attn_scale * log2(e)
  int kc;               // keys per LDS chunk (multiple of kStep)
  int row;              // K/V LDS row stride in elements
  int lrow;             // L tile row stride in floats
  int groups;           // task groups (workgroups) per query region
  int units;            // B * R * groups
  int per_xcd;          // ceil(units / 8)
  int accumulate;       // add the existing contents of out
};

template <bool BF16>
struct Elem;
template <>
struct Elem<true> { using T = uint16_t; };
template <>
struct Elem<false> { using T = float; };

// 8 consecutive elements -> MFMA operand slots (bf16: one 8-wide vector).
template <bool BF16>
struct Operand;

template <>
struct Operand<true> {
  bf16x8 v;
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = __builtin_bit_cast(bf16x8, *(const uint4*)p);
  }
  __device__ __forceinline__ void zero() { v = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }
};

template <>
struct Operand<false> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = *(const float4*)p;
    const float4 b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
};

__device__ __forceinline__ f32x4 mma(const Operand<true>& a, const Operand<true>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const Operand<false>& a, const Operand<false>& b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

// key offset (within a 32-key step) of operand slot e for lane group lg
__device__ __forceinline__ int slot_key(int lg, int e) {
  return e < 4 ? 4 * lg + e : 16 + 4 * lg + (e - 4);
}

template <bool BF16, int KS>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttnArgs A) {
  using T = typename Elem<BF16>::T;
  constexpr int VEC = 16 / (int)sizeof(T);
  extern __shared__ uint4 smem_attn[];
  const Shape& s = A.s;

  // XCD-aware unit order: consecutive units (same image) land on one XCD.
  const int unit = (blockIdx.x % kXcds) * A.per_xcd + blockIdx.x / kXcds;
  if (unit >= A.units) return;
  const int grp = unit % A.groups;
  const int br = unit / A.groups;
  const int b = br / s.R, r = br - b * s.R;
  const int ry = r / s.S, rx = r - ry * s.S;

  T* Ks = (T*)smem_attn;
  T* Vs = Ks + (size_t)A.kc * A.row;
  const T* __restrict__ Q = (const T*)A.q;
  const T* __restrict__ K = (const T*)A.k;
  const T* __restrict__ V = (const T*)A.v;
  const int32_t* __restrict__ irow = A.idx + (size_t)br * s.topk;

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lq = lane & 15;     // query column of this lane / key row of an operand
  const int lg = lane >> 4;     // 0..3
  const int nqb = (s.n + 15) / 16;
  const int ntasks = nqb * s.heads;

  // per-task register state
  Operand<BF16> qop[kTasksPerWave];
  f32x4 acc0[kTasksPerWave], acc1[kTasksPerWave];
  float m_run[kTasksPerWave], l_run[kTasksPerWave];
  int t_head[kTasksPerWave], t_q[kTasksPerWave];
  bool t_ok[kTasksPerWave];

#pragma unroll
  for (int i = 0; i < kTasksPerWave; ++i) {
    const int task = grp * kTasksPerBlock + i * kWaves + wave;
    t_ok[i] = task < ntasks;
    const int qb = t_ok[i] ? task / s.heads : 0;
    t_head[i] = t_ok[i] ? task - qb * s.heads : 0;
    t_q[i] = qb * 16 + lq;                // query token index in the region
    if (t_ok[i] && t_q[i] < s.n) {
      const int ty = t_q[i] / s.ws, tx = t_q[i] - ty * s.ws;
      qop[i].load(Q + pixel_offset(b, ry * s.hs + ty, rx * s.ws + tx, s) +
                  t_head[i] * kHeadDim + 8 * lg);
    } else {
      qop[i].zero();
    }
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }

  const int total = s.topk * s.n;
  const int G = s.C / VEC;
  for (int c0 = 0; c0 < total; c0 += A.kc) {
    const int kcnt = min(A.kc, total - c0);
    const int kpad = (kcnt + kStep - 1) / kStep * kStep;
    __syncthreads();
    for (int e = threadIdx.x; e < kpad * G; e += kThreads) {
      const int key = e / G, g = e - key * G;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < kcnt) {
        const int t = c0 + key;
        const int j = t / s.n, tok = t - j * s.n;
        int reg = irow[j];
        reg = min(max(reg, 0), s.R - 1);
        const int sy = reg / s.S, sx = reg - sy * s.S;
        const int ty = tok / s.ws, tx = tok - ty * s.ws;
        const size_t off = pixel_offset(b, sy * s.hs + ty, sx * s.ws + tx, s) + (size_t)g * VEC;
        kv = *(const uint4*)(K + off);
        vv = *(const uint4*)(V + off);
      }
      *(uint4*)(Ks + (size_t)key * A.row + g * VEC) = kv;
      *(uint4*)(Vs + (size_t)key * A.row + g * VEC) = vv;
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kTasksPerWave; ++i) {
      if (!t_ok[i]) continue;
      const int hoff = t_head[i] * kHeadDim;
      for (int ks = 0; ks < kpad; ks += kStep) {
        // S^T blocks: keys ks + lq (block 0) and ks + 16 + lq (block 1) as A rows
        Operand<BF16> ka, kb;
        ka.load(Ks + (size_t)(ks + lq) * A.row + hoff + 8 * lg);
        kb.load(Ks + (size_t)(ks + 16 + lq) * A.row + hoff + 8 * lg);
        const f32x4 s0 = mma(ka, qop[i], f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 s1 = mma(kb, qop[i], f32x4{0.f, 0.f, 0.f, 0.f});
        // lane holds keys ks + slot_key(lg, e), query lq
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = s0[e] * A.scale_log2;
          x[4 + e] = s1[e] * A.scale_log2;
        }
        if (ks + kStep > kcnt) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (ks + slot_key(lg, e) >= kcnt) x[e] = -INFINITY;
        }
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mt = fmaxf(mt, x[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m_run[i], mt);
        const float alpha = exp2f(m_run[i] - mn);
        m_run[i] = mn;
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2f(x[e] - mn);
          ps += p[e];
        }
        l_run[i] = l_run[i] * alpha + ps;
        acc0[i] *= alpha;
        acc1[i] *= alpha;
        // V^T operands: row d = lq (va) and 16 + lq (vb), same key slots as P^T
        if constexpr (BF16) {
          uint16_t ta[8], tb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const T* vr = Vs + (size_t)(ks + slot_key(lg, e)) * A.row + hoff;
            ta[e] = vr[lq];
            tb[e] = vr[16 + lq];
          }
          Operand<true> va, vb, phi, plo;
          va.v = as_bf16x8(ta[0] | ((uint32_t)ta[1] << 16), ta[2] | ((uint32_t)ta[3] << 16),
                           ta[4] | ((uint32_t)ta[5] << 16), ta[6] | ((uint32_t)ta[7] << 16));
          vb.v = as_bf16x8(tb[0] | ((uint32_t)tb[1] << 16), tb[2] | ((uint32_t)tb[3] << 16),
                           tb[4] | ((uint32_t)tb[5] << 16), tb[6] | ((uint32_t)tb[7] << 16));
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
            l[e] = pack_bf16x2(p[2 * e] - bf16_lo(h[e]), p[2 * e + 1] - bf16_hi(h[e]));
          }
          phi.v = as_bf16x8(h[0], h[1], h[2], h[3]);
          plo.v = as_bf16x8(l[0], l[1], l[2], l[3]);
          acc0[i] = mma(va, phi, acc0[i]);   // O^T rows d = 4*lg + e
          acc0[i] = mma(va, plo, acc0[i]);
          acc1[i] = mma(vb, phi, acc1[i]);   // O^T rows d = 16 + 4*lg + e
          acc1[i] = mma(vb, plo, acc1[i]);
        } else {
          Operand<false> va, vb, pop;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pop.v[e] = p[e];
            const T* vr = Vs + (size_t)(ks + slot_key(lg, e)) * A.row + hoff;
            va.v[e] = vr[lq];
            vb.v[e] = vr[16 + lq];
          }
          acc0[i] = mma(va, pop, acc0[i]);
          acc1[i] = mma(vb, pop, acc1[i]);
        }
      }
    }
  }

  float* Ls = nullptr;
  if constexpr (KS > 0) {
    // fused LePE: V halo tile, weights and the fp32 L tile in the staging area
    const size_t halo_elems = (size_t)(s.hs + KS - 1) * (s.ws + KS - 1) * s.C;
    T* Hs = (T*)smem_attn;
    float* Wt = (float*)(Hs + halo_elems);
    Ls = Wt + KS * KS * s.C;
    __syncthreads();
    stage_halo<BF16, KS>(A.v, A.w, b, ry * s.hs, rx * s.ws, s.hs, s.ws, 0, s.C, s, Hs, Wt);
    __syncthreads();
    conv_tile<BF16, KS>(Hs, Wt, A.bias, 0, s.hs, s.ws, s.C,
        [&](int y, int x, int c, float v0, float v1) {
          *(float2*)(Ls + (size_t)(y * s.ws + x) * A.lrow + c) = make_float2(v0, v1);
        });
    __syncthreads();
  }

  // normalise and store: lane holds query lq, channels 4*lg..+3 and 16+4*lg..+3
#pragma unroll
  for (int i = 0; i < kTasksPerWave; ++i) {
    if (!t_ok[i]) continue;
    float lt = l_run[i];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (t_q[i] >= s.n) continue;
    const float inv = 1.f / lt;
    const int ty = t_q[i] / s.ws, tx = t_q[i] - ty * s.ws;
    const size_t o = pixel_offset(b, ry * s.hs + ty, rx * s.ws + tx, s) + t_head[i] * kHeadDim;
    float r0[4], r1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = acc0[i][e] * inv;
      r1[e] = acc1[i][e] * inv;
    }
    if constexpr (KS > 0) {
      const float* lp = Ls + (size_t)t_q[i] * A.lrow + t_head[i] * kHeadDim;
      const float4 a0 = *(const float4*)(lp + 4 * lg);
      const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
      r0[0] += a0.x; r0[1] += a0.y; r0[2] += a0.z; r0[3] += a0.w;
      r1[0] += a1.x; r1[1] += a1.y; r1[2] += a1.z; r1[3] += a1.w;
    }
    if (A.accumulate) {
      float e0[4], e1[4];
      load4<BF16>(A.out, o + 4 * lg, e0);
      load4<BF16>(A.out, o + 16 + 4 * lg, e1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r0[e] += e0[e];
        r1[e] += e1[e];
      }
    }
    store4<BF16>(A.out, o + 4 * lg, r0);
    store4<BF16>(A.out, o + 16 + 4 * lg, r1);
  }
}

// ---------------------------------------------------------------------------
// Standalone LePE: out = L (ACCUM false) or out += L (ACCUM true), L as in
// conv_tile.  One workgroup per output tile of kLepeRows rows by kLepeCols
// columns and one slice of up to 64 channels; the zero-padded V tile and the
// slice's weights are staged in LDS with 16-byte loads, then convolved.
// ---------------------------------------------------------------------------
constexpr int kLepeCols = 16;

struct LepeGrid {
  int cs;       // channels per slice (64 or 32)
  int tiles_y;  // row tiles per image
};

template <bool BF16, int KS, bool ACCUM>
__global__ __launch_bounds__(kThreads) void lepe_kernel(
    const void* __restrict__ v, const float* __restrict__ w,
    const float* __restrict__ bias, void* __restrict__ out, Shape s, LepeGrid lg) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  extern __shared__ uint4 smem_lepe[];
  const int cs = lg.cs;
  const int c0 = blockIdx.z * cs;
  const int x0 = blockIdx.x * kLepeCols;
  const int b = blockIdx.y / lg.tiles_y;
  const int y0 = (blockIdx.y - b * lg.tiles_y) * kLepeRows;
  const int th = min(kLepeRows, s.H - y0), tw = min(kLepeCols, s.W - x0);
  T* Hs = (T*)smem_lepe;
  float* Wt = (float*)(Hs + (size_t)(kLepeRows + KS - 1) * (kLepeCols + KS - 1) * cs);
  stage_halo<BF16, KS>(v, w, b, y0, x0, th, tw, c0, cs, s, Hs, Wt);
  __syncthreads();
  conv_tile<BF16, KS>(Hs, Wt, bias, c0, th, tw, cs,
      [&](int y, int x, int c, float v0, float v1) {
        const size_t off = pixel_offset(b, y0 + y, x0 + x, s) + c0 + c;
        if constexpr (ACCUM) {
          float e[2];
          load2<BF16>(out, off, e);
          v0 += e[0];
          v1 += e[1];
        }
        if constexpr (BF16) {
          *(uint32_t*)((uint16_t*)out + off) = pack_bf16x2(v0, v1);
        } else {
          *(float2*)((float*)out + off) = make_float2(v0, v1);
        }
      });
}

template <bool BF16, int KS, bool ACCUM>
hipError_t lepe_launch_ks(const void* v, const float* w, const float* b, const Shape& s,
                          void* out, hipStream_t st) {
  LepeGrid lg;
  lg.cs = (s.C % 64 == 0) ? 64 : 32;
  lg.tiles_y = (s.H + kLepeRows - 1) / kLepeRows;
  const dim3 grid((unsigned)((s.W + kLepeCols - 1) / kLepeCols), (unsigned)(s.B * lg.tiles_y),
                  (unsigned)(s.C / lg.cs));
  const size_t esz = BF16 ? 2 : 4;
  const size_t lds = (size_t)(kLepeRows + KS - 1) * (kLepeCols + KS - 1) * lg.cs * esz +
                     (size_t)KS * KS * lg.cs * sizeof(float);
  const void* fn = (const void*)lepe_kernel<BF16, KS, ACCUM>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lepe_kernel<BF16, KS, ACCUM>), grid, dim3(kThreads), lds, st, v, w, b, out,
                     s, lg);
  return hipGetLastError();
}

template <bool BF16, bool ACCUM>
hipError_t lepe_launch(const void* v, const float* w, const float* b, int ks, const Shape& s,
                       void* out, hipStream_t st) {
  switch (ks) {
    case 1: return lepe_launch_ks<BF16, 1, ACCUM>(v, w, b, s, out, st);
    case 3: return lepe_launch_ks<BF16, 3, ACCUM>(v, w, b, s, out, st);
    case 5: return lepe_launch_ks<BF16, 5, ACCUM>(v, w, b, s, out, st);
    case 7: return lepe_launch_ks<BF16, 7, ACCUM>(v, w, b, s, out, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int KS>
hipError_t attend_launch_ks(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const void* fn = (const void*)attend_kernel<BF16, KS>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_kernel<BF16, KS>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t attend_launch(const AttnArgs& a, int ks, dim3 grid, size_t lds, hipStream_t st) {
  switch (ks) {
    case 0: return attend_launch_ks<BF16, 0>(a, grid, lds, st);
    case 1: return attend_launch_ks<BF16, 1>(a, grid, lds, st);
    case 3: return attend_launch_ks<BF16, 3>(a, grid, lds, st);
    case 5: return attend_launch_ks<BF16, 5>(a, grid, lds, st);
    case 7: return attend_launch_ks<BF16, 7>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_pool(const void* q, const void* k, double* qm, double* km, const Shape& s,
                       bool bf16, hipStream_t st) {
  const dim3 grid((unsigned)(s.B * s.R));
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(kThreads), 0, st, (const uint4*)q,
                       (const uint4*)k, qm, km, s);
  else
    hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(kThreads), 0, st, (const uint4*)q,
                       (const uint4*)k, qm, km, s);
  return hipGetLastError();
}

hipError_t launch_route(const double* qm, const double* km, const Shape& s, double route_scale,
                        int32_t* idx, float* logits, hipStream_t st) {
  const int nrb = (s.R + kRouteRows - 1) / kRouteRows;
  const size_t lds = (size_t)kRouteRows * (s.C + s.R) * sizeof(double);
  // wavefront arg-max rounds cost ~ topk*(J + 30); rank counting ~ J*R
  const int J = (s.R + 63) / 64;
  const int use_select = (long long)s.topk * (J + 30) < (long long)J * s.R ? 1 : 0;
  const hipError_t e = hipFuncSetAttribute((const void*)route_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)(s.B * nrb)), dim3(kThreads), lds, st, qm, km,
                     s, route_scale, idx, logits, use_select);
  return hipGetLastError();
}

hipError_t launch_attend(const void* q, const void* k, const void* v, const int32_t* idx,
                         const Shape& s, bool bf16, float attn_scale, const float* w,
                         const float* bias, int ks, void* out, hipStream_t st) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.idx = idx; a.out = out; a.w = w; a.bias = bias; a.s = s;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.accumulate = 0;
  const int esz = bf16 ? 2 : 4;
  const int vec = 16 / esz;
  a.row = s.C + vec;                                     // 16-byte pad per row
  a.lrow = s.C + 4;
  const size_t budget = 64 * 1024;
  int kc = (int)(budget / ((size_t)2 * a.row * esz)) / kStep * kStep;
  if (kc < kStep) kc = kStep;
  const int total = s.topk * s.n;
  const int total_pad = (total + kStep - 1) / kStep * kStep;
  if (kc > total_pad) kc = total_pad;
  a.kc = kc;
  const int ntasks = ((s.n + 15) / 16) * s.heads;
  a.groups = (ntasks + kTasksPerBlock - 1) / kTasksPerBlock;
  a.units = s.B * s.R * a.groups;
  a.per_xcd = (a.units + kXcds - 1) / kXcds;
  size_t lds = (size_t)2 * kc * a.row * esz;
  const dim3 grid((unsigned)(a.per_xcd * kXcds));
  int fused_ks = 0;
  if (w) {
    const size_t halo = (size_t)(s.hs + ks - 1) * (s.ws + ks - 1) * s.C * esz +
                        (size_t)ks * ks * s.C * sizeof(float) + (size_t)s.n * a.lrow * sizeof(float);
    if (a.groups == 1 && halo <= (lds > budget ? lds : budget)) {
      fused_ks = ks;
      if (halo > lds) lds = halo;
    } else {
      // LePE first (out = L), then attention adds its result into out
      const hipError_t e = bf16 ? lepe_launch<true, false>(v, w, bias, ks, s, out, st)
                                : lepe_launch<false, false>(v, w, bias, ks, s, out, st);
      if (e != hipSuccess) return e;
      a.accumulate = 1;
    }
  }
  return bf16 ? attend_launch<true>(a, fused_ks, grid, lds, st)
              : attend_launch<false>(a, fused_ks, grid, lds, st);
}

hipError_t launch_lepe(const void* v, const float* w, const float* b, int ks, const Shape& s,
                       bool bf16, void* out, hipStream_t st) {
  return bf16 ? lepe_launch<true, true>(v, w, b, ks, s, out, st)
              : lepe_launch<false, true>(v, w, b, ks, s, out, st);
}

}  // namespace bra
