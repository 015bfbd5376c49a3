// Region pooling and routing kernels of the BRA forward pass (gfx950).
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析",
// p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的
// 计算范式".

#include <climits>
#include <type_traits>

#include "device_common.h"

namespace bra {
namespace {

// ---------------------------------------------------------------------------
// Pool: region means of Q and K in float64 (p1 §3 region-mean step; p2 §2
// mean over the region-internal axes).
//
// 32 lanes (half a wavefront) per region, 8 regions per workgroup.  A lane
// owns one 16-byte channel group (gl lanes per pixel, gl the largest power
// of two <= min(groups, 32); wider pixels take several passes) and a strided
// subset of the region's pixels, whose loads it issues in batches.  The
// partial sums of the 32/gl pixel lanes are then added across lanes with
// row rotations (DPP) and a row swap (v_permlane16_swap): no LDS, no
// barrier, and a fixed order, so the result is deterministic.  Summing bf16
// or f32 values in float64 is exact or within one rounding of the exact
// sum, so routing sees the same means as a float64 reference.
// ---------------------------------------------------------------------------
constexpr int kPoolBatch = 4;
constexpr int kRegionsPerPoolBlock = kThreads / 32;

struct PoolArgs {
  const uint4* q;
  const uint4* k;
  double* qm;
  double* km;
  Shape s;
  int gl;          // lanes per pixel (power of two, <= 32)
  int units;       // B * R
  int rpw;         // regions per wavefront (pool_pipe_kernel)
  FastDiv f_ws, f_R, f_S;
};

// Row rotation by SH lanes (DPP row_ror), applied to both halves of a double.
template <int SH>
__device__ __forceinline__ double ror_row(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x120 | SH, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x120 | SH, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// The value of lane l ^ 16 (rows swapped in pairs).
__device__ __forceinline__ double xor16d(double v) {
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)__double2loint(v), (unsigned)__double2loint(v), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap((unsigned)__double2hiint(v), (unsigned)__double2hiint(v), false, false);
  const bool up = threadIdx.x & 16;
  return __hiloint2double((int)(up ? b[0] : b[1]), (int)(up ? a[0] : a[1]));
}

// Sum over the lanes of a 32-lane half that share lane % gl.
__device__ __forceinline__ double half_sum(double v, int gl) {
  if (gl <= 1) v += ror_row<1>(v);
  if (gl <= 2) v += ror_row<2>(v);
  if (gl <= 4) v += ror_row<4>(v);
  if (gl <= 8) v += ror_row<8>(v);
  if (gl <= 16) v += xor16d(v);
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs A) {
  constexpr int VEC = BF16 ? 8 : 4;
  const Shape& s = A.s;
  const int br = blockIdx.x * kRegionsPerPoolBlock + (threadIdx.x >> 5);
  if (br >= A.units) return;                 // no barrier follows
  const int l32 = threadIdx.x & 31;
  const int b = fdiv(br, A.f_R), r = br - b * s.R;
  const int ry = fdiv(r, A.f_S), rx = r - ry * s.S;
  const int G = s.C / VEC;                   // 16-byte groups per pixel
  const int gl = A.gl, PL = 32 / gl;
  const int pl = l32 / gl, gi = l32 - pl * gl;
  const double inv_n = 1.0 / (double)s.n;
  const uint4* __restrict__ q = A.q + (size_t)b * s.H * s.W * G;
  const bool two = A.k != nullptr;                // else: means of q only
  const uint4* __restrict__ k = two ? A.k + (size_t)b * s.H * s.W * G : nullptr;
  const int base = (ry * s.hs * s.W + rx * s.ws) * G;
  for (int g0 = 0; g0 < G; g0 += gl) {
    const int g = g0 + gi;
    const bool gok = g < G;
    double aq[VEC], ak[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) { aq[e] = 0.0; ak[e] = 0.0; }
    for (int t0 = pl; t0 < s.n; t0 += kPoolBatch * PL) {
      uint4 uq[kPoolBatch], uk[kPoolBatch];
#pragma unroll
      for (int u = 0; u < kPoolBatch; ++u) {
        const int t = t0 + u * PL;
        uq[u] = make_uint4(0, 0, 0, 0);
        uk[u] = make_uint4(0, 0, 0, 0);
        if (gok && t < s.n) {
          const int ty = fdiv(t, A.f_ws), tx = t - ty * s.ws;
          const int off = base + (ty * s.W + tx) * G + g;
          uq[u] = q[off];
          if (two) uk[u] = k[off];
        }
      }
#pragma unroll
      for (int u = 0; u < kPoolBatch; ++u) {
        float fq[VEC], fk[VEC];
        unpack16<BF16>(uq[u], fq);
        unpack16<BF16>(uk[u], fk);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { aq[e] += (double)fq[e]; ak[e] += (double)fk[e]; }
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      aq[e] = half_sum(aq[e], gl);
      ak[e] = half_sum(ak[e], gl);
    }
    if (pl == 0 && gok) {
      const size_t o = (size_t)br * s.C + (size_t)g * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        A.qm[o + e] = aq[e] * inv_n;
        if (two) A.km[o + e] = ak[e] * inv_n;
      }
    }
  }
}

// Bandwidth-first pooling for pixels of G <= 64 16-byte groups (G a power of
// two): one wavefront per region, lane (p, g) = (lane / G, lane % G) owns
// channel group g of pixels p, p + 64/G, ...; every load of a batch of up to
// kWavePass passes (two tensors; eight passes cover an 8x8 region of
// 128-byte pixels in one batch) is issued before the first add, as buffer
// loads with no branch (tokens past the region read zero).  The float64
// partial sums of the 64/G lanes sharing g are then added with row rotations
// and row swaps, in a fixed order.
#ifndef BRA_POOL_NPMAX
#define BRA_POOL_NPMAX 8
#endif
#ifndef BRA_POOL_WAVES
#define BRA_POOL_WAVES 4
#endif
constexpr int kPoolWaves = BRA_POOL_WAVES;      // wavefronts (regions) per workgroup
constexpr int kWavePass = BRA_POOL_NPMAX;


template <int SH>
__device__ __forceinline__ double ror_rowd(double v) { return ror_row<SH>(v); }

__device__ __forceinline__ double xor32d(double v) {
  const auto a = __builtin_amdgcn_permlane32_swap((unsigned)__double2loint(v), (unsigned)__double2loint(v), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap((unsigned)__double2hiint(v), (unsigned)__double2hiint(v), false, false);
  const bool up = threadIdx.x & 32;
  return __hiloint2double((int)(up ? b[0] : b[1]), (int)(up ? a[0] : a[1]));
}

// Sum over the lanes of the wavefront that share lane % G.
template <int G>
__device__ __forceinline__ double group_sum(double v) {
  if constexpr (G <= 1) v += ror_row<1>(v);
  if constexpr (G <= 2) v += ror_row<2>(v);
  if constexpr (G <= 4) v += ror_row<4>(v);
  if constexpr (G <= 8) v += ror_row<8>(v);
  if constexpr (G <= 16) v += xor16d(v);
  if constexpr (G <= 32) v += xor32d(v);
  return v;
}

template <bool BF16, int G, int NP, bool TWO>
__global__ __launch_bounds__(kPoolWaves * 64) void pool_wave_kernel(PoolArgs A) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int PP = 64 / G;                 // pixels per pass
  const Shape& s = A.s;
  // the wavefront's region, uniform by construction (readfirstlane tells the
  // compiler so: the buffer descriptors below then live in scalar registers)
  const int br = __builtin_amdgcn_readfirstlane(blockIdx.x * kPoolWaves + (threadIdx.x >> 6));
  if (br >= A.units) return;                 // no barrier follows
  const int lane = threadIdx.x & 63, g = lane % G, p0 = lane / G;
  const int b = fdiv(br, A.f_R), r = br - b * s.R;
  const int ry = fdiv(r, A.f_S), rx = r - ry * s.S;
  // buffer loads: a token past the region reads zero at an offset past the
  // record, so every load of a batch is issued unconditionally
  const uint32_t img_bytes = (uint32_t)s.H * s.W * G * 16;
  const auto qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(A.q + (size_t)b * s.H * s.W * G), (short)0, (int)img_bytes, 0x00020000);
  const auto kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(TWO ? A.k + (size_t)b * s.H * s.W * G : A.q), (short)0, (int)img_bytes,
      0x00020000);
  const int base = (ry * s.hs * s.W + rx * s.ws) * G + g;
  double aq[VEC], ak[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { aq[e] = 0.0; ak[e] = 0.0; }
  for (int t0 = p0; t0 < s.n; t0 += NP * PP) {
    uint4 uq[NP], uk[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int t = t0 + u * PP;
      const int ty = fdiv(t, A.f_ws), tx = t - ty * s.ws;
      const uint32_t off = t < s.n ? (uint32_t)(base + (ty * s.W + tx) * G) * 16 : 0x80000000u;
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t vq = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
      uq[u] = make_uint4(vq.x, vq.y, vq.z, vq.w);
      if constexpr (TWO) {
        const u32x4_t vk = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
        uk[u] = make_uint4(vk.x, vk.y, vk.z, vk.w);
      } else {
        uk[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      float fq[VEC], fk[VEC];
      unpack16<BF16>(uq[u], fq);
      if constexpr (TWO) unpack16<BF16>(uk[u], fk);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        aq[e] += (double)fq[e];
        if constexpr (TWO) ak[e] += (double)fk[e];
      }
    }
  }
  const double inv_n = 1.0 / (double)s.n;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    aq[e] = group_sum<G>(aq[e]);
    if constexpr (TWO) ak[e] = group_sum<G>(ak[e]);
  }
  if (p0 == 0) {
    const size_t o = (size_t)br * s.C + (size_t)g * VEC;
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      *(double2*)(A.qm + o + e) = make_double2(aq[e] * inv_n, aq[e + 1] * inv_n);
      if constexpr (TWO) *(double2*)(A.km + o + e) = make_double2(ak[e] * inv_n, ak[e + 1] * inv_n);
    }
  }
}

// Pipelined pooling for pixels of G in {8, 16, 32, 64} 16-byte groups whose
// region fits one batch of passes: each wavefront takes rpw consecutive
// regions.  Lane (p, g) = (lane / G, lane % G) owns group g of pixels p,
// p + 64/G, ...  As soon as pass u of region r has been added, the load of
// pass u of region r + 1 goes out into the same registers, so the float64
// adds of one region overlap the loads of the next.  The last region issues
// no loads, so none is in flight when the wavefront ends.
//
// The float64 partial sums of the 64/G lanes that share g are combined by a
// reduce-scatter over lane bits 5, 4, 3 (as far as they index pixels): at
// each step a lane pair exchanges half of its values, so the lane with the
// bit clear ends with the pair's sums of the lower half and its partner with
// those of the upper half.  Bits 5 and 4 use the row-swap permutes, which move
// both halves in one instruction; bit 3 a DPP row rotation.  Afterwards lane
// (p, g) holds values p*KEEP .. p*KEEP + KEEP - 1 of its group (value index
// = tensor * VEC + channel), fully summed in a fixed order, and stores them.
// Offsets are 32-bit over the whole tensor (the launcher checks its size).
// ---------------------------------------------------------------------------

// Exchange within lane pairs differing in bit BIT: the lane with the bit
// clear returns x + x', the lane with it set y + y' (primes: the partner's).
template <int BIT>
__device__ __forceinline__ double pair_keep(double x, double y) {
  if constexpr (BIT == 5 || BIT == 4) {
    const unsigned xl = (unsigned)__double2loint(x), xh = (unsigned)__double2hiint(x);
    const unsigned yl = (unsigned)__double2loint(y), yh = (unsigned)__double2hiint(y);
    // vdst's upper half (rows 1, 3) trades places with src0's lower half
    // (rows 0, 2): a clear lane ends with (own x, partner's x), a set lane
    // with (partner's y, own y)
    const auto l = BIT == 5 ? __builtin_amdgcn_permlane32_swap(xl, yl, false, false)
                            : __builtin_amdgcn_permlane16_swap(xl, yl, false, false);
    const auto h = BIT == 5 ? __builtin_amdgcn_permlane32_swap(xh, yh, false, false)
                            : __builtin_amdgcn_permlane16_swap(xh, yh, false, false);
    return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
  } else {
    static_assert(BIT == 3, "pixel lanes start at bit 3 or above");
    const bool up = threadIdx.x & 8;
    const double send = up ? x : y, keep = up ? y : x;
    return keep + ror_row<8>(send);       // row rotation by 8 = lane ^ 8
  }
}

template <int BIT, int M>
__device__ __forceinline__ void scatter_step(double* v) {
#pragma unroll
  for (int i = 0; i < M / 2; ++i) v[i] = pair_keep<BIT>(v[i], v[i + M / 2]);
}

template <bool BF16, int G, int NP, bool TWO>
__global__ __launch_bounds__(kPoolWaves * 64) void pool_pipe_kernel(PoolArgs A) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int PP = 64 / G;                 // pixels per pass = lanes sharing g
  constexpr int NT = TWO ? 2 : 1;
  constexpr int NV = NT * VEC;               // values per lane
  constexpr int KEEP = NV / PP;              // values per lane after the scatter
  static_assert(G >= 8 && G <= 64 && KEEP >= 1, "shape handled by pool_wave_kernel");
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const Shape& s = A.s;
  const int wv = __builtin_amdgcn_readfirstlane(blockIdx.x * kPoolWaves + (threadIdx.x >> 6));
  const int r0 = wv * A.rpw;
  if (r0 >= A.units) return;                 // no barrier follows
  const int r1 = min(r0 + A.rpw, A.units);
  const int lane = threadIdx.x & 63, g = lane % G, p = lane / G;
  const uint32_t bytes = (uint32_t)s.B * s.H * s.W * G * 16;
  const auto qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(A.q), (short)0, (int)bytes,
                                                    0x00020000);
  const auto kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(TWO ? A.k : A.q), (short)0,
                                                    (int)bytes, 0x00020000);
  // this lane's token offsets within a region (bytes); tokens past the
  // region get an offset past any record
  uint32_t toff[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int t = p + u * PP;
    const int ty = fdiv(t, A.f_ws), tx = t - ty * s.ws;
    toff[u] = t < s.n ? (uint32_t)(((ty * s.W + tx) * G + g) * 16) : 0x80000000u;
  }
  // byte offset of region br's first pixel
  auto region_base = [&](int br) -> uint32_t {
    const int b = fdiv(br, A.f_R), r = br - b * s.R;
    const int ry = fdiv(r, A.f_S), rx = r - ry * s.S;
    return (uint32_t)(((b * s.H + ry * s.hs) * s.W + rx * s.ws) * G * 16);
  };
  uint4 bq[NP], bk[NP];
  auto issue = [&](int u, uint32_t base) {
    const uint32_t off = base + toff[u];
    const u32x4_t vq = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
    bq[u] = make_uint4(vq.x, vq.y, vq.z, vq.w);
    if constexpr (TWO) {
      const u32x4_t vk = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      bk[u] = make_uint4(vk.x, vk.y, vk.z, vk.w);
    }
  };
  {
    const uint32_t base = region_base(r0);
#pragma unroll
    for (int u = 0; u < NP; ++u) issue(u, base);
  }
  const double inv_n = 1.0 / (double)s.n;
  // one region: add its passes (handing each pass's registers to the next
  // region's load when NEXT), then reduce and store
  auto region = [&](int br, auto next) {
    constexpr bool NEXT = decltype(next)::value;
    const uint32_t nbase = NEXT ? region_base(br + 1) : 0u;
    double v[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) v[e] = 0.0;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      float f[VEC];
      unpack16<BF16>(bq[u], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] += (double)f[e];
      if constexpr (TWO) {
        unpack16<BF16>(bk[u], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[VEC + e] += (double)f[e];
      }
      if constexpr (NEXT) issue(u, nbase);
    }
    if constexpr (PP >= 2) scatter_step<5, NV>(v);
    if constexpr (PP >= 4) scatter_step<4, NV / 2>(v);
    if constexpr (PP >= 8) scatter_step<3, NV / 4>(v);
    // lane p holds values p*KEEP .. p*KEEP + KEEP - 1
#pragma unroll
    for (int j = 0; j < KEEP; j += (KEEP >= 2 ? 2 : 1)) {
      const int o = p * KEEP + j;
      const int tsr = o / VEC, e = o - tsr * VEC;
      double* dst = (tsr ? A.km : A.qm) + (size_t)br * s.C + g * VEC + e;
      if constexpr (KEEP >= 2)
        *(double2*)dst = make_double2(v[j] * inv_n, v[j + 1] * inv_n);
      else
        *dst = v[j] * inv_n;
    }
  };
  for (int br = r0; br + 1 < r1; ++br) region(br, std::true_type());
  region(r1 - 1, std::false_type());
}

// ---------------------------------------------------------------------------
// Route: A[r][s] = route_scale * <q_r[r], k_r[s]> in float64, then per row
// the topk largest entries, largest first, equal values by lower index (p1
// §3 affinity and top-k; p2 §4 scaled affinity and top-k).
//
// One workgroup per (image, block of 16 rows).  The 16 x R affinity strip is
// a small float64 GEMM on the matrix cores (v_mfma_f64_16x16x4, 16 x 16
// column tiles dealt to the wavefronts); each lane feeds 4 consecutive
// channels as the K elements of 4 successive MFMAs, so one 32-byte read
// serves 4 steps.  The block's query-region rows come from LDS, staged once
// for all wavefronts; each wavefront loads only its own tiles' key rows.
// The strip lives in LDS only; nothing of A is written to memory.  Ranking
// runs topk rounds of an arg-max per row over a group of L = 16, 32 or 64
// lanes (the narrowest that holds R in 16 candidates a lane: 4, 2 or 1 rows
// per wavefront), each lane first picking its best untaken candidate, then
// DPP row rotations and row swaps across the group, no LDS.  For R <= 64,
// route_small_kernel ranks either that way or by counting (rank(s) = number
// of entries ranking before s).  Both rank through an order-preserving int64
// key (after turning -0 into +0, so that 0 and -0 tie, as they compare
// equal), equal keys by lower index, and give the same answer.
// ---------------------------------------------------------------------------
constexpr int kRouteRows = 16;
#ifndef BRA_ROUTE_WAVES
#define BRA_ROUTE_WAVES 16
#endif
constexpr int kRouteWaves = BRA_ROUTE_WAVES;   // wavefronts of a route_kernel workgroup
constexpr int kRouteTiles = 1024 / 16 / kRouteWaves;   // column tiles a wavefront, R <= 1024
constexpr int kRouteQs = 66;      // LDS row stride of the staged query rows (doubles): the 16
                                  // rows' 32-byte reads fall in distinct banks

__device__ __forceinline__ long long order_key(double v) {
  v = v + 0.0;                                   // -0 -> +0
  const long long k = __double_as_longlong(v);
  return k ^ ((k >> 63) & 0x7fffffffffffffffLL);
}

// true if (ka, ia) ranks before (kb, ib)
__device__ __forceinline__ bool ranks_before(long long ka, int ia, long long kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// (key, index) of another lane, moved by a DPP row rotation or a row swap.
template <int SH>
__device__ __forceinline__ void ror_pair(long long& k, int& i) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)k, 0x120 | SH, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(k >> 32), 0x120 | SH, 0xf, 0xf, false);
  const int ii = __builtin_amdgcn_update_dpp(0, i, 0x120 | SH, 0xf, 0xf, false);
  k = ((long long)hi << 32) | (unsigned)lo;
  i = ii;
}

// All lanes of each group of L lanes (L = 16, 32 or 64, groups aligned) end
// with the (key, index) ranking first over the group: rotations inside each
// 16-lane row, then, for wider groups, swaps between rows.
template <int L>
__device__ __forceinline__ void group_best(long long& bk, int& bi) {
#define BRA_ROW_STEP(SH)                                  \
  {                                                       \
    long long ok = bk;                                    \
    int oi = bi;                                          \
    ror_pair<SH>(ok, oi);                                 \
    if (ranks_before(ok, oi, bk, bi)) { bk = ok; bi = oi; } \
  }
  BRA_ROW_STEP(8)
  BRA_ROW_STEP(4)
  BRA_ROW_STEP(2)
  BRA_ROW_STEP(1)
#undef BRA_ROW_STEP
  if constexpr (L >= 32) {
    const bool up16 = threadIdx.x & 16;
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)bk, (unsigned)bk, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((unsigned)(bk >> 32), (unsigned)(bk >> 32), false, false);
    const auto x = __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    const long long ok = ((long long)(up16 ? h[0] : h[1]) << 32) | (up16 ? a[0] : a[1]);
    const int oi = (int)(up16 ? x[0] : x[1]);
    if (ranks_before(ok, oi, bk, bi)) { bk = ok; bi = oi; }
  }
  if constexpr (L == 64) {
    const bool up32 = threadIdx.x & 32;
    const auto a = __builtin_amdgcn_permlane32_swap((unsigned)bk, (unsigned)bk, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((unsigned)(bk >> 32), (unsigned)(bk >> 32), false, false);
    const auto x = __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false);
    const long long ok = ((long long)(up32 ? h[0] : h[1]) << 32) | (up32 ? a[0] : a[1]);
    const int oi = (int)(up32 ? x[0] : x[1]);
    if (ranks_before(ok, oi, bk, bi)) { bk = ok; bi = oi; }
  }
}

__device__ __forceinline__ void wave_best(long long& bk, int& bi) { group_best<64>(bk, bi); }

struct RouteArgs {
  const double* qm;
  const double* km;
  int32_t* idx;
  float* logits;
  Shape s;
  double scale;
  int lda;          // LDS row stride of the affinity strip (doubles)
  int nrb;          // row blocks per image
};

template <int L, int JT>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(RouteArgs A) {
  extern __shared__ double strip[];                // [kRouteRows][lda], staged rows
  const Shape& s = A.s;
  const int R = s.R, C = s.C, topk = s.topk;
  const int b = blockIdx.x / A.nrb, r0 = (blockIdx.x - b * A.nrb) * kRouteRows;
  const int rows = min(kRouteRows, R - r0);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int l16 = lane & 15, lk = lane >> 4;

  // affinity strip on the matrix cores.  The strip's 16 query-region rows
  // are staged once per 64-channel chunk into LDS (every wavefront reads
  // them); each wavefront keeps the accumulators of its column tiles (at
  // most kRouteTiles) across the chunks and loads its tiles' key rows itself
  double* qs = strip + kRouteRows * A.lda;          // [16][kRouteQs]
  const double* __restrict__ qimg = A.qm + (size_t)b * R * C;
  const double* __restrict__ kimg = A.km + (size_t)b * R * C;
  const int ntile = (R + 15) / 16;
  f64x4 acc[kRouteTiles];
#pragma unroll
  for (int t = 0; t < kRouteTiles; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < C; c0 += 64) {
    {
      const int row = threadIdx.x >> 6, ch = threadIdx.x & 63;   // 16 x 64, one a thread
      const int rr = min(r0 + row, R - 1);
      qs[row * kRouteQs + ch] = c0 + ch < C ? qimg[(size_t)rr * C + c0 + ch] : 0.0;
    }
    __syncthreads();
    // lane group lk supplies channels c + 4*lk .. c + 4*lk + 3 (c = c0 + 16*u)
    // over 4 steps; a tile's 8 loads are issued before its MFMAs
#pragma unroll
    for (int t = 0; t < kRouteTiles; ++t) {
      const int ct = wave + t * kRouteWaves;
      if (ct >= ntile) break;                                     // wave-uniform
      const double* kp = kimg + (size_t)min(ct * 16 + l16, R - 1) * C + 4 * lk;
      double4 a4[4], b4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = c0 + 16 * u;
        b4[u] = cc + 4 * lk < C ? *(const double4*)(kp + cc) : make_double4(0.0, 0.0, 0.0, 0.0);
        a4[u] = *(const double4*)(qs + l16 * kRouteQs + 16 * u + 4 * lk);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].x, b4[u].x, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].y, b4[u].y, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].z, b4[u].z, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].w, b4[u].w, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();                                              // qs is restaged next
  }
  // D layout (f64 16x16x4): lane holds column l16 of the tile, rows lk + 4*i
#pragma unroll
  for (int t = 0; t < kRouteTiles; ++t) {
    const int ct = wave + t * kRouteWaves;
    if (ct >= ntile) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = lk + 4 * i, cc = ct * 16 + l16;
      if (rr < rows && cc < R) strip[rr * A.lda + cc] = A.scale * acc[t][i];
    }
  }
  __syncthreads();

  // ranking: a group of L lanes per strip row, 64 / L rows per wavefront;
  // lane li of a group holds candidates li, li + L, ... (JT slots), in
  // increasing index order, so within a lane a strictly larger key is the
  // only way to rank before the current best
  constexpr int RPW = 64 / L;
  if (wave * RPW >= rows) return;                  // wave-uniform; no barrier follows
  const int rl = wave * RPW + lane / L, li = lane % L;
  const bool live = rl < rows;
  const double* ar = strip + min(rl, rows - 1) * A.lda;
  long long keys[JT];
  unsigned taken = 0;                              // bit j: slot j taken or empty
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int sc = li + L * j;
    keys[j] = sc < R ? order_key(ar[sc]) : LLONG_MIN;
    if (sc >= R) taken |= 1u << j;
  }
  int32_t* irow = A.idx + ((size_t)b * R + r0 + rl) * topk;
  float* lrow = A.logits ? A.logits + ((size_t)b * R + r0 + rl) * topk : nullptr;
  for (int kk = 0; kk < topk; ++kk) {
    long long bk = LLONG_MIN;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int sc = li + L * j;
      if (!((taken >> j) & 1u) && ranks_before(keys[j], sc, bk, bi)) {
        bk = keys[j];
        bi = sc;
      }
    }
    group_best<L>(bk, bi);
    if ((bi & (L - 1)) == li) taken |= 1u << (bi / L);
    if (li == 0 && live) {
      irow[kk] = bi;
      if (lrow) lrow[kk] = (float)ar[bi];
    }
  }
}

// Route for R <= 64 regions (one candidate per lane).  One 16-wavefront
// workgroup per (image, 16-row strip).  Wavefront w computes column tile
// w % 4 of the strip over channel quarter w / 4 (v_mfma_f64_16x16x4f64, its
// loads all issued before the first MFMA); the four partial strips of each
// tile are added in LDS, in a fixed order.  Then wavefront w ranks strip row
// w: for topk <= 2 by topk rounds of a wavefront arg-max, otherwise by
// counting (each lane counts the candidates of its row that rank before its
// own, keys broadcast from LDS, and the lanes of rank < topk write
// themselves).  Sixteen wavefronts per CU hide the load and MFMA latency.
constexpr int kSmallWaves = 16;
constexpr int kSelectMaxK = 2;    // arg-max rounds up to this topk, rank counting above
constexpr int kSmallMaxC4 = 4;     // double4 loads per operand and lane (C <= 256 per pass)

__global__ __launch_bounds__(kSmallWaves * 64) void route_small_kernel(RouteArgs A) {
  __shared__ double part[4][kRouteRows][64];
  __shared__ long long keys[kRouteRows][64];
  const Shape& s = A.s;
  const int R = s.R, C = s.C, topk = s.topk;
  const int b = blockIdx.x / A.nrb, r0 = (blockIdx.x - b * A.nrb) * kRouteRows;
  const int rows = min(kRouteRows, R - r0);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int l16 = lane & 15, lk = lane >> 4;
  const int tile = wave & 3, quarter = wave >> 2;
  const double* __restrict__ qimg = A.qm + (size_t)b * R * C;
  const double* __restrict__ kimg = A.km + (size_t)b * R * C;
  const int ntile = (R + 15) / 16;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  if (tile < ntile) {
    const double* qp = qimg + (size_t)min(r0 + l16, R - 1) * C + 4 * lk;
    const double* kp = kimg + (size_t)min(16 * tile + l16, R - 1) * C + 4 * lk;
    // channel groups of 16 of this quarter: c = 16 * (quarter + 4 * u)
    for (int c0 = 16 * quarter; c0 < C; c0 += 64 * kSmallMaxC4) {
      double4 a4[kSmallMaxC4], b4[kSmallMaxC4];
#pragma unroll
      for (int u = 0; u < kSmallMaxC4; ++u) {
        const int c = c0 + 64 * u;
        const bool ok = c + 4 * lk < C;
        a4[u] = ok ? *(const double4*)(qp + c) : make_double4(0.0, 0.0, 0.0, 0.0);
        b4[u] = ok ? *(const double4*)(kp + c) : make_double4(0.0, 0.0, 0.0, 0.0);
      }
#pragma unroll
      for (int u = 0; u < kSmallMaxC4; ++u) {
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].x, b4[u].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].y, b4[u].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].z, b4[u].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[u].w, b4[u].w, acc, 0, 0, 0);
      }
    }
    // D layout (f64 16x16x4): lane holds column l16 of the tile, rows lk + 4*i
#pragma unroll
    for (int i = 0; i < 4; ++i) part[quarter][lk + 4 * i][16 * tile + l16] = acc[i];
  }
  __syncthreads();

  const int rl = wave;
  if (rl >= rows) return;                          // no barrier follows
  const double v =
      ((part[0][rl][lane] + part[1][rl][lane]) + (part[2][rl][lane] + part[3][rl][lane])) * A.scale;
  const long long key = lane < R ? order_key(v) : LLONG_MIN;
  if (topk <= kSelectMaxK) {
    // topk rounds of a wavefront arg-max over the candidates not yet taken
    bool taken = lane >= R;
    for (int kk = 0; kk < topk; ++kk) {
      long long bk = taken ? LLONG_MIN : key;
      int bi = taken ? 0x7fffffff : lane;
      wave_best(bk, bi);
      if (lane == bi) {
        taken = true;
        const size_t o = ((size_t)b * R + r0 + rl) * topk + kk;
        A.idx[o] = lane;
        if (A.logits) A.logits[o] = (float)v;
      }
    }
    return;
  }
  // rank of this candidate = number of candidates ranking before it; every
  // lane reads each key of its row (one LDS broadcast per candidate)
  keys[rl][lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // the row's keys are visible
  int rank = 0;
#pragma unroll 8
  for (int s2 = 0; s2 < R; ++s2) rank += ranks_before(keys[rl][s2], s2, key, lane) ? 1 : 0;
  if (lane < R && rank < topk) {
    const size_t o = ((size_t)b * R + r0 + rl) * topk + rank;
    A.idx[o] = lane;
    if (A.logits) A.logits[o] = (float)v;
  }
}

// ---------------------------------------------------------------------------
// Pool and route in one launch, for R <= 64 regions: one 16-wavefront
// workgroup per (image, strip of at most 16 rows) pools the float64 means of all the
// image's K regions and of its strip's Q regions into LDS, then forms the
// strip's affinities and ranks them as route_small_kernel does.  Each strip
// pools the image's K itself (the image's strips share one XCD, so the
// repeated reads come from its L2): no second launch, no wait between
// workgroups, and the means reach the affinity without a round trip through
// memory.  When asked for (qm, km not null) they are also written out (K by
// the first strip, Q by every strip for its rows) for callers that read
// them; the forward pass does not ask, which saves writing float64 means as
// large as the bf16 inputs at 2x2-pixel regions.
//
// Pooling: wavefront w takes items w, w + 16, ... (K regions 0..R-1, then
// the strip's Q regions); lane (p, g) = (lane / G, lane % G) owns 16-byte
// channel group g of pixels p, p + 64/G, ...; IB items' loads are in flight
// at once in a ring of registers, refilled as each item is added (a region
// of more than 8 passes takes 2 or 4 slots in turn, one band of its pixel
// rows each, its sums carried from one to the next); the
// float64 partial sums of the 64/G lanes sharing g are combined by the
// reduce-scatter of pool_pipe_kernel, in a fixed order.
// ---------------------------------------------------------------------------
struct PoolRouteArgs {
  const uint4* q;
  const uint4* k;
  double* qm;
  double* km;
  int32_t* idx;
  float* logits;
  Shape s;
  double scale;
  int nrb;          // 16-row strips per image
  int ldm;          // LDS row stride of the means (doubles)
  int gr;           // 16-byte groups of a pixel (G, or fewer: the lanes of g >= gr idle)
  int parts_log2;   // a region's pixels in 2^parts_log2 runs of NP passes (one ring slot each)
  uint32_t part_off;  // bytes from one run to the next (whole pixel rows)
  FastDiv f_ws, f_S;
};

template <bool BF16, int G, int NP, int IB>
__global__ __launch_bounds__(kSmallWaves * 64) void pool_route_kernel(PoolRouteArgs A) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int PP = 64 / G;                 // pixels per pass = lanes sharing g
  constexpr int KEEP = VEC / PP;             // values per lane after the scatter
  static_assert(G >= 1 && G <= 64 && KEEP >= 1, "pixel lanes in bits log2(G)..5");
  extern __shared__ double pr_lds[];
  const Shape& s = A.s;
  const int R = s.R, C = s.C, topk = s.topk;
  // workgroup -> (image, strip): the strips of an image sit on its XCD
  const int xcd = blockIdx.x % kXcds, rest = blockIdx.x / kXcds;
  const int t1 = rest / A.nrb, strip = rest - t1 * A.nrb;
  const int b = t1 * kXcds + xcd;
  if (b >= s.B) return;                      // uniform; before any barrier
  // the image's rows split evenly over its nrb strips (at most 16 each), so
  // that no workgroup pools more than R + ceil(R / nrb) regions: at R = 49,
  // 62 items (at most four a wavefront) rather than 16 + 49 = 65
  const int r0 = strip * R / A.nrb;
  const int rows = (strip + 1) * R / A.nrb - r0;
  // the wavefront index as a scalar: items, and so the buffer descriptor
  // each load takes, are uniform over the wavefront
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, lk = lane >> 4;
  double* means = pr_lds;                    // [R + 16][ldm]: K regions, then the strip's Q

  // ---- pool ----
  {
    // a pixel's gr groups on G lanes (G the power of two at or above gr):
    // the lanes of g >= gr load nothing and keep nothing
    const int g = lane % G, p = lane / G;
    const int gr = A.gr;
    const bool gok = g < gr;
    const uint32_t img_bytes = (uint32_t)s.H * s.W * gr * 16;
    const size_t img = (size_t)b * s.H * s.W * gr;
    const auto Qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(A.q + img), (short)0,
                                                      (int)img_bytes, 0x00020000);
    const auto Kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(A.k + img), (short)0,
                                                      (int)img_bytes, 0x00020000);
    uint32_t toff[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int t = p + u * PP;
      const int ty = fdiv(t, A.f_ws), tx = t - ty * s.ws;
      toff[u] = t < s.n && gok ? (uint32_t)(((ty * s.W + tx) * gr + g) * 16) : 0x80000000u;
    }
    // ring entry j is run j % 2^ps of the wavefront's item j / 2^ps
    const int ps = A.parts_log2, H = 1 << ps;
    const int U = R + rows;
    const int ni = wave < U ? (U - wave + kSmallWaves - 1) / kSmallWaves : 0;
    const int nj = ni << ps;
    uint4 buf[IB][NP];
    auto issue = [&](int slot, int j) {
      const int item = wave + kSmallWaves * (j >> ps);
      const int reg = item < R ? item : r0 + item - R;
      const int ry = fdiv(reg, A.f_S), rx = reg - ry * s.S;
      const uint32_t base = (uint32_t)(((ry * s.hs) * s.W + rx * s.ws) * gr * 16) +
                            (uint32_t)(j & (H - 1)) * A.part_off;
      const auto rs = item < R ? Kr : Qr;       // uniform over the wavefront
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, base + toff[u], 0, 0);
        buf[slot][u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    };
#pragma unroll
    for (int sl = 0; sl < IB; ++sl)
      if (sl < nj) issue(sl, sl);
    const double inv_n = 1.0 / (double)s.n;
    double v[VEC];                               // an item's sums, over its runs
    for (int j0 = 0; j0 < nj; j0 += IB) {
#pragma unroll
      for (int sl = 0; sl < IB; ++sl) {
        const int j = j0 + sl;
        if (j >= nj) break;                      // uniform
        const int item = wave + kSmallWaves * (j >> ps);
        if ((j & (H - 1)) == 0) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = 0.0;
        }
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          float f[VEC];
          unpack16<BF16>(buf[sl][u], f);
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] += (double)f[e];
        }
        if (j + IB < nj) issue(sl, j + IB);
        if ((j & (H - 1)) != H - 1) continue;   // uniform: more runs of this item to come
        if constexpr (PP >= 2) scatter_step<5, VEC>(v);
        if constexpr (PP >= 4) scatter_step<4, VEC / 2>(v);
        if constexpr (PP >= 8) scatter_step<3, VEC / 4>(v);
        // lane p holds values p*KEEP .. p*KEEP + KEEP - 1 of group g
        const int row = item;                    // K regions first, then the strip's Q rows
        double* gdst = !A.qm ? nullptr
                     : item < R ? (strip == 0 ? A.km + ((size_t)b * R + item) * C : nullptr)
                                : A.qm + ((size_t)b * R + r0 + item - R) * C;
        if (gok) {
#pragma unroll
          for (int jj = 0; jj < KEEP; ++jj) {
            const int c = g * VEC + p * KEEP + jj;
            const double m = v[jj] * inv_n;
            means[row * A.ldm + c] = m;
            if (gdst) gdst[c] = m;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- affinity strip: wavefront w, column tile w % 4 over channel quarter w / 4 ----
  const int tile = wave & 3, quarter = wave >> 2;
  const int ntile = (R + 15) / 16;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  if (tile < ntile) {
    const double* qp = means + (R + min(l16, rows - 1)) * A.ldm + 4 * lk;
    const double* kp = means + min(16 * tile + l16, R - 1) * A.ldm + 4 * lk;
    for (int c0 = 16 * quarter; c0 < C; c0 += 64) {
      const bool ok = c0 + 4 * lk < C;
      const double4 a4 = ok ? *(const double4*)(qp + c0) : make_double4(0.0, 0.0, 0.0, 0.0);
      const double4 b4 = ok ? *(const double4*)(kp + c0) : make_double4(0.0, 0.0, 0.0, 0.0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4.x, b4.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4.y, b4.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4.z, b4.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a4.w, b4.w, acc, 0, 0, 0);
    }
  }
  __syncthreads();                           // the means are read; their space is reused
  double (*part)[kRouteRows][64] = (double (*)[kRouteRows][64])pr_lds;
  long long (*keys)[64] = (long long (*)[64])(pr_lds + 4 * kRouteRows * 64);
  if (tile < ntile) {
    // D layout (f64 16x16x4): lane holds column l16 of the tile, rows lk + 4*i
#pragma unroll
    for (int i = 0; i < 4; ++i) part[quarter][lk + 4 * i][16 * tile + l16] = acc[i];
  }
  __syncthreads();

  // ---- ranking of strip row w (as route_small_kernel) ----
  const int rl = wave;
  if (rl >= rows) return;                    // no barrier follows
  const double v =
      ((part[0][rl][lane] + part[1][rl][lane]) + (part[2][rl][lane] + part[3][rl][lane])) * A.scale;
  const long long key = lane < R ? order_key(v) : LLONG_MIN;
  const size_t orow = ((size_t)b * R + r0 + rl) * topk;
  if (topk <= kSelectMaxK) {
    bool taken = lane >= R;
    for (int kk = 0; kk < topk; ++kk) {
      long long bk = taken ? LLONG_MIN : key;
      int bi = taken ? 0x7fffffff : lane;
      wave_best(bk, bi);
      if (lane == bi) {
        taken = true;
        A.idx[orow + kk] = lane;
        if (A.logits) A.logits[orow + kk] = (float)v;
      }
    }
    return;
  }
  keys[rl][lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // the row's keys are visible
  int rank = 0;
#pragma unroll 8
  for (int s2 = 0; s2 < R; ++s2) rank += ranks_before(keys[rl][s2], s2, key, lane) ? 1 : 0;
  if (lane < R && rank < topk) {
    A.idx[orow + rank] = lane;
    if (A.logits) A.logits[orow + rank] = (float)v;
  }
}

template <bool BF16, int G, int NP>
hipError_t pool_route_launch(const PoolRouteArgs& a, size_t lds, hipStream_t st) {
  constexpr int IB = NP >= 8 ? 1 : 8 / NP;   // ring of IB items: 32 VGPRs of loads
  const void* fn = reinterpret_cast<const void*>(&pool_route_kernel<BF16, G, NP, IB>);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.s.B + kXcds - 1) / kXcds * kXcds * a.nrb));
  hipLaunchKernelGGL((pool_route_kernel<BF16, G, NP, IB>), grid, dim3(kSmallWaves * 64), lds, st,
                     a);
  return hipGetLastError();
}

// Launches pool_pipe_kernel for shapes it covers (one value or more per lane
// after the scatter); the launcher never selects the others.
template <bool BF16, int G, int NP, bool TWO>
void launch_pool_pipe(dim3 grid, const PoolArgs& a, hipStream_t st) {
  if constexpr ((BF16 ? 8 : 4) * (TWO ? 2 : 1) >= 64 / G)
    hipLaunchKernelGGL((pool_pipe_kernel<BF16, G, NP, TWO>), grid, dim3(kPoolWaves * 64), 0, st, a);
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, double* qm, double* km, const Shape& s,
                       bool bf16, hipStream_t st) {
  PoolArgs a;
  a.q = (const uint4*)q; a.k = (const uint4*)k; a.qm = qm; a.km = km; a.s = s;
  const int G = s.C / (bf16 ? 8 : 4);
  a.gl = 1;
  while (a.gl * 2 <= G && a.gl * 2 <= 32) a.gl *= 2;
  a.units = s.B * s.R;
  a.f_ws = make_fastdiv(s.ws);
  a.f_R = make_fastdiv(s.R);
  a.f_S = make_fastdiv(s.S);
  const int nv = (bf16 ? 8 : 4) * (k ? 2 : 1);
  const bool pipe_g = G == 8 || G == 16 || G == 32 || G == 64;
  const int passes_pipe = pipe_g ? (s.n + 64 / G - 1) / (64 / G) : 0;
  // the pipelined kernel: offsets over the whole tensor below 2^31, pixel
  // lanes in bits 3..5, at least one value per lane after the scatter, and a
  // region read in one batch
  if (pipe_g && nv >= 64 / G && passes_pipe <= kWavePass &&
      (long long)s.B * s.H * s.W * G * 16 < 0x80000000LL) {
    // two regions per wavefront once there are enough regions to fill the
    // chip twice over (on MI355X the 64-image 56x56 stage-1 shape then pools
    // and routes in 16.9 us against 17.1 with one); with few regions, one
    // each keeps more wavefronts busy
    a.rpw = a.units >= 2048 ? 2 : 1;
    const int np = passes_pipe > 4 ? 8 : passes_pipe > 2 ? 4 : passes_pipe > 1 ? 2 : 1;
    const long long waves = (a.units + a.rpw - 1) / a.rpw;
    const dim3 pgrid((unsigned)((waves + kPoolWaves - 1) / kPoolWaves));
#define BRA_PIPE_LAUNCH(BB, GG, NN, TT) launch_pool_pipe<BB, GG, NN, TT>(pgrid, a, st)
#define BRA_PIPE_NP(GG, NN)                                                                   \
    if (G == GG && np == NN) {                                                               \
      if (bf16) {                                                                            \
        if (k) BRA_PIPE_LAUNCH(true, GG, NN, true); else BRA_PIPE_LAUNCH(true, GG, NN, false);   \
      } else {                                                                               \
        if (k) BRA_PIPE_LAUNCH(false, GG, NN, true); else BRA_PIPE_LAUNCH(false, GG, NN, false); \
      }                                                                                      \
      return hipGetLastError();                                                              \
    }
#define BRA_PIPE_G(GG) BRA_PIPE_NP(GG, 1) BRA_PIPE_NP(GG, 2) BRA_PIPE_NP(GG, 4) BRA_PIPE_NP(GG, 8)
    BRA_PIPE_G(8) BRA_PIPE_G(16) BRA_PIPE_G(32) BRA_PIPE_G(64)
#undef BRA_PIPE_G
#undef BRA_PIPE_NP
#undef BRA_PIPE_LAUNCH
  }
  // the wavefront kernel's buffer offsets within an image stay below 2^31
  if (G <= 64 && (G & (G - 1)) == 0 && (long long)s.H * s.W * G * 16 < 0x80000000LL) {
    // passes per load batch: just enough for the region (at most kWavePass)
    const int passes = (s.n + 64 / G - 1) / (64 / G);
    const int np = passes >= kWavePass ? kWavePass : passes > 2 ? 4 : passes > 1 ? 2 : 1;
    const dim3 wgrid((unsigned)((a.units + kPoolWaves - 1) / kPoolWaves));
#define BRA_POOL_LAUNCH(BB, GG, NN, TT) \
    hipLaunchKernelGGL((pool_wave_kernel<BB, GG, NN, TT>), wgrid, dim3(kPoolWaves * 64), 0, st, a)
#define BRA_POOL_NP(GG, NN)                                                                   \
    if (G == GG && np == NN) {                                                               \
      if (bf16) {                                                                            \
        if (k) BRA_POOL_LAUNCH(true, GG, NN, true); else BRA_POOL_LAUNCH(true, GG, NN, false);   \
      } else {                                                                               \
        if (k) BRA_POOL_LAUNCH(false, GG, NN, true); else BRA_POOL_LAUNCH(false, GG, NN, false); \
      }                                                                                      \
      return hipGetLastError();                                                              \
    }
#define BRA_POOL_G(GG) BRA_POOL_NP(GG, 1) BRA_POOL_NP(GG, 2) BRA_POOL_NP(GG, 4) BRA_POOL_NP(GG, 8)
    BRA_POOL_G(1) BRA_POOL_G(2) BRA_POOL_G(4) BRA_POOL_G(8) BRA_POOL_G(16) BRA_POOL_G(32)
    BRA_POOL_G(64)
#undef BRA_POOL_G
#undef BRA_POOL_NP
#undef BRA_POOL_LAUNCH
  }
  const dim3 grid((unsigned)((a.units + kRegionsPerPoolBlock - 1) / kRegionsPerPoolBlock));
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_route(const double* qm, const double* km, const Shape& s, double route_scale,
                        int32_t* idx, float* logits, hipStream_t st) {
  RouteArgs a;
  a.qm = qm; a.km = km; a.idx = idx; a.logits = logits; a.s = s; a.scale = route_scale;
  a.nrb = (s.R + kRouteRows - 1) / kRouteRows;
  a.lda = (s.R + 15) / 16 * 16 + 1;
  if (s.R <= 64) {
    hipLaunchKernelGGL(route_small_kernel, dim3((unsigned)(s.B * a.nrb)), dim3(kSmallWaves * 64), 0,
                       st, a);
    return hipGetLastError();
  }
  // lanes per ranking row: the narrowest group holding R in 16 candidates
  // a lane (R <= 1024 is checked by the callers)
  const int L = s.R <= 256 ? 16 : s.R <= 512 ? 32 : 64;
  const int J = (s.R + L - 1) / L;
  const void* fn = L == 16 ? (J <= 8 ? (const void*)route_kernel<16, 8> : (const void*)route_kernel<16, 16>)
                 : L == 32 ? (const void*)route_kernel<32, 16> : (const void*)route_kernel<64, 16>;
  const size_t lds = ((size_t)kRouteRows * a.lda + (size_t)kRouteRows * kRouteQs) * sizeof(double);
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(s.B * a.nrb)), block(kRouteWaves * 64);
  if (L == 16 && J <= 8)
    hipLaunchKernelGGL((route_kernel<16, 8>), grid, block, lds, st, a);
  else if (L == 16)
    hipLaunchKernelGGL((route_kernel<16, 16>), grid, block, lds, st, a);
  else if (L == 32)
    hipLaunchKernelGGL((route_kernel<32, 16>), grid, block, lds, st, a);
  else
    hipLaunchKernelGGL((route_kernel<64, 16>), grid, block, lds, st, a);
  return hipGetLastError();
}

hipError_t launch_pool_route(const void* q, const void* k, double* qm, double* km, const Shape& s,
                             bool bf16, double route_scale, int32_t* idx, float* logits,
                             hipStream_t st) {
  const int vec = bf16 ? 8 : 4;
  if (s.R > 64 || s.C % vec) return hipErrorNotSupported;
  const int gr = s.C / vec;
  // lanes a pixel: the power of two at or above its 16-byte groups (a
  // quarter of them idle at C = 96 in bf16)
  int G = 8;
  while (G < gr) G *= 2;
  if (G > 64) return hipErrorNotSupported;
  const int PP = 64 / G;
  if (vec < PP) return hipErrorNotSupported;                 // a value a lane after the scatter
  const int passes = (s.n + PP - 1) / PP;
  // more than 8 passes: the region in 2 or 4 runs of 8 passes (whole rows
  // of the region each), one ring slot a run, so that a lane holds no more
  // than 32 VGPRs of loads (C = 96 and 128 at 8x8-pixel regions: 2 runs)
  int parts_log2 = 0;
  if (passes > 8) {
    const int run = 8 * PP;                    // pixels a run
    if (s.n % run || run % s.ws) return hipErrorNotSupported;
    const int parts = s.n / run;
    if (parts != 2 && parts != 4) return hipErrorNotSupported;
    parts_log2 = parts == 2 ? 1 : 2;
  }
  if ((long long)s.H * s.W * gr * 16 >= 0x80000000LL) return hipErrorNotSupported;
  int dev = 0, lds_max = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  PoolRouteArgs a;
  a.q = (const uint4*)q; a.k = (const uint4*)k; a.qm = qm; a.km = km;
  a.idx = idx; a.logits = logits; a.s = s; a.scale = route_scale;
  a.nrb = (s.R + kRouteRows - 1) / kRouteRows;
  if (parts_log2) {
    // runs double a workgroup's round trips to memory: worth it only while
    // the launch has a workgroup for every CU (64 images of 56x56 at C = 96:
    // forward 77.6-81.3 -> 70.2-71.8 us; 16 images of 64x64 at C = 128, 64
    // workgroups: 53.1-55.4 -> 67.8-70.0 us, so the two launches stay there)
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if ((long long)s.B * a.nrb < cus) return hipErrorNotSupported;
  }
  a.ldm = s.C + 2;              // 16 bytes of padding: the 16 rows' reads spread over the banks
  a.gr = gr;
  a.parts_log2 = parts_log2;
  a.part_off = parts_log2 ? (uint32_t)((8 * PP / s.ws) * s.W * gr * 16) : 0u;
  a.f_ws = make_fastdiv(s.ws);
  a.f_S = make_fastdiv(s.S);
  size_t lds = (size_t)(s.R + kRouteRows) * a.ldm * sizeof(double);
  const size_t rank_lds = (size_t)(4 * kRouteRows * 64 + kRouteRows * 64) * sizeof(double);
  if (lds < rank_lds) lds = rank_lds;
  if (lds > (size_t)lds_max) return hipErrorNotSupported;
  const int np = passes > 4 ? 8 : passes > 2 ? 4 : passes > 1 ? 2 : 1;
#define BRA_PR(BB, GG)                                                   \
  if (G == GG) {                                                         \
    switch (np) {                                                        \
      case 1: return pool_route_launch<BB, GG, 1>(a, lds, st);           \
      case 2: return pool_route_launch<BB, GG, 2>(a, lds, st);           \
      case 4: return pool_route_launch<BB, GG, 4>(a, lds, st);           \
      default: return pool_route_launch<BB, GG, 8>(a, lds, st);          \
    }                                                                    \
  }
  if (bf16) {
    BRA_PR(true, 8) BRA_PR(true, 16) BRA_PR(true, 32) BRA_PR(true, 64)
  } else {
    BRA_PR(false, 16) BRA_PR(false, 32) BRA_PR(false, 64)
  }
#undef BRA_PR
  return hipErrorNotSupported;
}

}  // namespace bra
