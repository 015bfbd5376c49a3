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

#include <type_traits>

namespace bra {
namespace {

constexpr int kLinRows = 128;     // tokens per workgroup (32 per wavefront)
constexpr int kLinCols = 64;      // output features per workgroup
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
  const void* r;        // residual [T, N] added before the rounding (EPI 2), or null
  void* y[3];           // output groups: columns [g*ng, (g+1)*ng) go to y[g], [T, ng]
  int ng;               // columns per output group
  int T, K, N;
  int col_tiles, row_tiles, per_xcd;
  int col_groups;       // workgroups per row tile (each takes a share of the feature tiles)
  int nbuf;             // W staging buffers (1 when a workgroup has one step)
};

// Y = X W^T + b on the matrix cores, computed as Y^T = W X^T so that a lane
// ends with 4 consecutive output features of one token (one 8- or 16-byte
// store).  A workgroup owns 128 tokens (wavefront w: tokens 32w .. 32w+31, two
// 16-token blocks) and walks all output features in tiles of 64 (four 16-row
// blocks of W), K in chunks of KCH columns.  Each (feature tile, chunk) step
// stages W's 64 x KCH block in LDS (16-byte chunks XOR-swizzled by row, two
// buffers), the next step's block being loaded into registers while the
// current one is multiplied.  X is read straight from memory in the operand
// layout (one 16-byte row segment per lane); when K fits one chunk it is
// read once and reused for every feature tile.  When there are few row
// tiles, the feature tiles of a row tile are shared among col_groups
// workgroups.  Work items go to XCDs in contiguous ranges.  The output tile
// of a wavefront (32 tokens x 64 features) goes through LDS so that each
// 128-byte line of a token's features is written by 8 adjacent lanes in one
// store.  Epilogue EPI: 0 bias only, 1 bias then GELU (exact erf form), 2
// bias then a residual tensor added; each rounds once to the output type.
// GELU: gelu_as in device_common.h.

template <int EPI>
__device__ __forceinline__ float lin_act(float v) {
  if constexpr (EPI == 1) return gelu_as(v);
  return v;
}

template <bool BF16, int KCH, int EPI>
__global__ __launch_bounds__(kThreads) void linear_kernel(LinArgs a) {
  constexpr int ES = BF16 ? 2 : 4;                 // element bytes
  constexpr int KSTEP = BF16 ? 32 : 4;             // k per MFMA
  constexpr int CE = 16 / ES;                      // elements per 16-byte chunk
  constexpr int NKS = KCH / KSTEP;                 // k-steps of a full chunk
  constexpr int XPL = BF16 ? 1 : 8;                // f32: 8 one-float k-steps per group
  constexpr int CPR = KCH / CE;                    // 16-byte chunks per staged row (full chunk)
  constexpr int WPT = kLinCols * CPR / kThreads;   // staged chunks per thread
  constexpr bool F32ST = EPI == 2 || !BF16;        // output tile staged in float32
  constexpr int SES = F32ST ? 4 : ES;
  constexpr int ORB = kLinCols * SES + 16;         // output staging row (padded)
  using XT = typename std::conditional<BF16, bf16x8, float>::type;
  extern __shared__ __align__(16) unsigned char lds[];
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int item = xcd * a.per_xcd + loc;
  if (loc >= a.per_xcd || item >= a.row_tiles * a.col_groups) return;   // uniform; no barrier yet
  const int rt = item / a.col_groups, cg = item - rt * a.col_groups;
  const int ct_per = (a.col_tiles + a.col_groups - 1) / a.col_groups;
  const int ct0 = cg * ct_per, ct1 = min(a.col_tiles, ct0 + ct_per);
  const int t0 = rt * kLinRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const auto X = lin_rsrc(a.x, (uint32_t)a.T * a.K * ES);
  const unsigned char* W = (const unsigned char*)a.w;
  const int nch = (a.K + KCH - 1) / KCH;
  const int nsteps = (ct1 - ct0) * nch;
  const int bufb = kLinCols * min(a.K, KCH) * ES;  // bytes of one W staging buffer
  unsigned char* ost = lds + a.nbuf * bufb + wave * 32 * ORB;   // this wavefront's output tile

  uint4 wv[WPT];
  auto load_w = [&](int step) {                    // W block of a step into registers
    const int ct = ct0 + step / nch, kc = (step % nch) * KCH;
    const int kn = min(KCH, a.K - kc), cpr = kn / CE;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / cpr, c = e - r * cpr;
      const int n = ct * kLinCols + r;
      wv[i] = make_uint4(0, 0, 0, 0);
      if (e < kLinCols * cpr && n < a.N)
        wv[i] = *(const uint4*)(W + ((size_t)n * a.K + kc + c * CE) * ES);
    }
  };
  XT xo[NKS / XPL][2][XPL];
  auto load_x = [&](int kc) {                      // this wavefront's X operands of a chunk
    const int kn = min(KCH, a.K - kc);
#pragma unroll
    for (int ks = 0; ks < NKS / XPL; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int u = 0; u < XPL; ++u) {
          const int kk = (ks * XPL + u) * KSTEP;
          const int t = t0 + 32 * wave + 16 * tb + lq;
          const bool ok = t < a.T && kk < kn;
          if constexpr (BF16) {
            const uint32_t off = ok ? ((uint32_t)t * a.K + kc + kk + 8 * lg) * 2 : kLinOob;
            xo[ks][tb][u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(X, off, 0, 0));
          } else {
            const uint32_t off = ok ? ((uint32_t)t * a.K + kc + kk + lg) * 4 : kLinOob;
            xo[ks][tb][u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(X, off, 0, 0));
          }
        }
  };

  load_w(0);
  if (nch == 1) load_x(0);                         // reused by every feature tile
  f32x4 acc[2][4];
  for (int step = 0; step < nsteps; ++step) {
    const int ct = ct0 + step / nch, ch = step % nch, kc = ch * KCH;
    const int kn = min(KCH, a.K - kc), cpr = kn / CE;
    const int sw = cpr % 8 == 0 ? 7 : 3;           // cpr is a multiple of 4
    unsigned char* buf = lds + (step & 1) * bufb;
    if (nch > 1) load_x(kc);
    // staged row r, chunk c at chunk c ^ (r & sw); the barrier of the
    // previous step ordered every read of this buffer (two steps ago) first
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / cpr, c = e - r * cpr;
      if (e < kLinCols * cpr) *(uint4*)(buf + (r * cpr + (c ^ (r & sw))) * 16) = wv[i];
    }
    __syncthreads();
    if (step + 1 < nsteps) load_w(step + 1);
    if (ch == 0) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < NKS / XPL; ++ks)
#pragma unroll
      for (int u = 0; u < XPL; ++u) {
        const int kk = (ks * XPL + u) * KSTEP;
        if (kk >= kn) continue;                    // uniform
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int r = 16 * nb + lq;
          if constexpr (BF16) {
            const int c = (kk >> 3) + lg;          // chunk of k = kk + 8 lg
            const bf16x8 wa = *(const bf16x8*)(buf + (r * cpr + (c ^ (r & sw))) * 16);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              acc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xo[ks][tb][u], acc[tb][nb], 0, 0, 0);
          } else {
            const int k = kk + lg, c = k >> 2;
            const float wa = *(const float*)(buf + (r * cpr + (c ^ (r & sw))) * 16 + (k & 3) * 4);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              acc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wa, xo[ks][tb][u], acc[tb][nb], 0, 0, 0);
          }
        }
      }
    if (ch != nch - 1) continue;
    // bias, one rounding, then the tile through this wavefront's LDS rows:
    // lane (lq, lg) holds Y[token 16tb + lq][features 16nb + 4lg + 0..3]
    const int n0 = ct * kLinCols;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + 16 * nb + 4 * lg;
      float bb[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.b && n < a.N) {                        // N % 4 == 0: all four or none
        const float4 bv = *(const float4*)(a.b + n);
        bb[0] = bv.x; bb[1] = bv.y; bb[2] = bv.z; bb[3] = bv.w;
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const f32x4 v = acc[tb][nb];
        unsigned char* d = ost + (16 * tb + lq) * ORB + (16 * nb + 4 * lg) * SES;
        const float o0 = lin_act<EPI>(v[0] + bb[0]), o1 = lin_act<EPI>(v[1] + bb[1]);
        const float o2 = lin_act<EPI>(v[2] + bb[2]), o3 = lin_act<EPI>(v[3] + bb[3]);
        if constexpr (F32ST) *(float4*)d = make_float4(o0, o1, o2, o3);
        else *(uint2*)d = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // 16-byte chunks of output: kLinCols * ES / 16 per token row, 64 lanes per store
    const int n_last = min(n0 + kLinCols, a.N) - 1;
    const int g_tile = __builtin_amdgcn_readfirstlane(n0 / a.ng);
    const bool one_group = g_tile == __builtin_amdgcn_readfirstlane(n_last / a.ng);
    constexpr int CPRO = kLinCols * ES / 16;
    constexpr int TPS = 64 / CPRO;                 // token rows per store
#pragma unroll
    for (int i = 0; i < 32 / TPS; ++i) {
      const int tr = TPS * i + lane / CPRO, ck = lane % CPRO;
      const unsigned char* sp = ost + tr * ORB + ck * CE * SES;
      uint4 v;
      const int t = t0 + 32 * wave + tr, n = n0 + ck * CE;
      const bool ok = n < a.N && t < a.T;
      if constexpr (EPI == 2) {
        // residual chunk at the same place of r ([T, N], one group)
        const auto R = lin_rsrc(a.r, (uint32_t)a.T * a.N * ES);
        const uint32_t roff = ok ? ((uint32_t)t * a.N + n) * ES : kLinOob;
        const u32x4 rv = __builtin_amdgcn_raw_buffer_load_b128(R, roff, 0, 0);
        float rf[CE];
        unpack16<BF16>(make_uint4(rv.x, rv.y, rv.z, rv.w), rf);
        if constexpr (BF16) {
          const float4 a0 = *(const float4*)sp, a1 = *(const float4*)(sp + 16);
          v = make_uint4(pack_bf16x2(a0.x + rf[0], a0.y + rf[1]), pack_bf16x2(a0.z + rf[2], a0.w + rf[3]),
                         pack_bf16x2(a1.x + rf[4], a1.y + rf[5]), pack_bf16x2(a1.z + rf[6], a1.w + rf[7]));
        } else {
          const float4 a0 = *(const float4*)sp;
          v = make_uint4(__float_as_uint(a0.x + rf[0]), __float_as_uint(a0.y + rf[1]),
                         __float_as_uint(a0.z + rf[2]), __float_as_uint(a0.w + rf[3]));
        }
      } else {
        v = *(const uint4*)sp;                     // bf16 staged, or float32 output
      }
      // a chunk lies in one group (ng is a multiple of 8 or the chunk is the
      // last, partial one of a single group: N % 8 == 4 in bf16).  When the
      // whole tile lies in one group (the usual case) the group is uniform
      // and its descriptor is built once in scalar registers; otherwise each
      // lane's group is used (the compiler then loops over the distinct ones)
      int g;
      if (one_group) g = g_tile;
      else g = ok ? n / a.ng : 0;
      const int col = n - g * a.ng;
      const auto Y = lin_rsrc(a.y[g], (uint32_t)a.T * a.ng * ES);
      const uint32_t off = ok ? ((uint32_t)t * a.ng + col) * ES : kLinOob;
      if (n + CE <= a.N) {
        const u32x4 p = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(p, Y, off, 0, 0);
      } else {                                     // 4 features left (bf16 only)
        const u32x2 p = {v.x, v.y};
        __builtin_amdgcn_raw_buffer_store_b64(p, Y, off, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // tile read before the next one
  }
}

// qm = xm Wq^T + bq and km = xm Wk^T + bk in float64 (Wq, Wk: rows 0..C-1
// and C..2C-1 of w_qkv) on v_mfma_f64_16x16x4f64.  A workgroup owns one
// 16-row tile of the means and 4 NT column tiles of 16 (of the 2C outputs);
// wavefront w takes column tiles w, w+4, ..., so each load of a row segment
// of xm feeds NT independent accumulators.  Each lane feeds CPL consecutive
// channels as the k slots of CPL successive MFMAs (the same permutation on
// both operands); the next step's operands are loaded while the current one
// is multiplied.  The launcher uses CPL = 8 (the module's C is heads of 32
// channels): a weight row arrives as 64-byte segments, half the requests of
// CPL = 4 (on MI355X the 14 x 14 x 256 module step went 111.3 -> 106.0 us).  NT is 1 for C <= 64 and 2 above: the launch is
// small (one workgroup per 16 regions and 4 NT tiles), so spreading the
// C / 4 dependent MFMAs of a tile over more wavefronts wins until the chains
// are long enough that sharing each xm load pays (on MI355X the module step
// on the 56 x 56 x 64 stage shape: 87.7 us with 4 tiles a wavefront, 83.7
// with 1; on the 14 x 14 x 256 one: 111.2 with 4, 109.6 with 2, 117.3 with 1).

struct MeansArgs {
  const double* xm;     // [rows, C]
  const void* w;        // w_qkv [3C, C]
  const float* b;       // b_qkv [3C] or null
  double* qm;           // [rows, C]
  double* km;           // [rows, C]
  int rows, C;
  int col_tiles, col_blocks;
};

template <bool BF16, int NT, int CPL>
__global__ __launch_bounds__(kThreads) void means_proj_kernel(MeansArgs a) {
  constexpr int STEP = 4 * CPL;                     // channels a step
  const int rt = blockIdx.x / a.col_blocks, cbk = blockIdx.x - rt * a.col_blocks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lk = lane >> 4;
  const int r0 = rt * 16;
  const int C = a.C;
  const double* xp = a.xm + (size_t)min(r0 + l16, a.rows - 1) * C + CPL * lk;
  int wn[NT];
  bool tok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int ct = cbk * NT * kWaves + wave + kWaves * j;
    tok[j] = ct < a.col_tiles;
    wn[j] = tok[j] ? ct * 16 + l16 : 0;
  }
  double xa[CPL];
  double wb[NT][CPL];
  auto load = [&](int c) {
#pragma unroll
    for (int q = 0; q < CPL / 4; ++q) {
      const double4 x4 = *(const double4*)(xp + c + 4 * q);
      xa[4 * q] = x4.x; xa[4 * q + 1] = x4.y; xa[4 * q + 2] = x4.z; xa[4 * q + 3] = x4.w;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (BF16) {
        const uint16_t* wp = (const uint16_t*)a.w + (size_t)wn[j] * C + c + CPL * lk;
        if constexpr (CPL == 8) {
          const uint4 w = *(const uint4*)wp;
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) { wb[j][2 * e] = bf16_lo(u[e]); wb[j][2 * e + 1] = bf16_hi(u[e]); }
        } else {
          const uint2 w = *(const uint2*)wp;
          wb[j][0] = bf16_lo(w.x); wb[j][1] = bf16_hi(w.x); wb[j][2] = bf16_lo(w.y); wb[j][3] = bf16_hi(w.y);
        }
      } else {
        const float* wp = (const float*)a.w + (size_t)wn[j] * C + c + CPL * lk;
#pragma unroll
        for (int q = 0; q < CPL / 4; ++q) {
          const float4 w = *(const float4*)(wp + 4 * q);
          wb[j][4 * q] = w.x; wb[j][4 * q + 1] = w.y; wb[j][4 * q + 2] = w.z; wb[j][4 * q + 3] = w.w;
        }
      }
    }
  };
  f64x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(0);
  for (int c = 0; c < C; c += STEP) {
    double xc[CPL], wc[NT][CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) xc[e] = xa[e];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < CPL; ++e) wc[j][e] = wb[j][e];
    if (c + STEP < C) load(c + STEP);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < CPL; ++e)
        acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(xc[e], wc[j][e], acc[j], 0, 0, 0);
  }
  // D layout (f64 16x16x4): lane holds column l16 of the tile, rows lk + 4i
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (!tok[j]) continue;
    const int n = wn[j];
    const double bias = a.b ? (double)a.b[n] : 0.0;
    double* dst = n < C ? a.qm : a.km;
    const int col = n < C ? n : n - C;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + lk + 4 * i;
      if (r < a.rows) dst[(size_t)r * C + col] = acc[j][i] + bias;
    }
  }
}

}  // namespace

hipError_t launch_linear(const void* x, int T, int K, const void* w, const float* b, int N,
                         void* const* y, int groups, bool bf16, hipStream_t st, int epi,
                         const void* resid) {
  if (T <= 0 || K <= 0 || N <= 0 || K % 32 || N % 4 || groups < 1 || groups > 3 ||
      N % groups || (N / groups) % (groups > 1 ? 8 : 4))
    return hipErrorInvalidValue;
  const int es = bf16 ? 2 : 4;
  // buffer offsets are 32-bit: every operand below 2 GiB
  if ((long long)T * K * es >= (long long)kLinOob || (long long)T * (N / groups) * es >= (long long)kLinOob)
    return hipErrorNotSupported;
  if (epi < 0 || epi > 2 || (epi == 2 && (!resid || groups != 1))) return hipErrorInvalidValue;
  LinArgs a;
  a.x = x; a.w = w; a.b = b; a.r = resid;
  for (int g = 0; g < 3; ++g) a.y[g] = g < groups ? y[g] : y[0];
  a.ng = N / groups;
  a.T = T; a.K = K; a.N = N;
  a.col_tiles = (N + kLinCols - 1) / kLinCols;
  a.row_tiles = (T + kLinRows - 1) / kLinRows;
  // K chunk: all of K up to 256 in bf16 (X read once), 64 for float32
  const int kch = !bf16 ? 64 : K <= 64 ? 64 : K <= 128 ? 128 : 256;
  const void* fn;
#define BRA_LIN_FN(BB, KK) \
  (epi == 0 ? (const void*)&linear_kernel<BB, KK, 0> \
            : epi == 1 ? (const void*)&linear_kernel<BB, KK, 1> : (const void*)&linear_kernel<BB, KK, 2>)
  if (bf16 && kch == 64) fn = BRA_LIN_FN(true, 64);
  else if (bf16 && kch == 128) fn = BRA_LIN_FN(true, 128);
  else if (bf16) fn = BRA_LIN_FN(true, 256);
  else fn = BRA_LIN_FN(false, 64);
#undef BRA_LIN_FN
  const size_t orb = (size_t)kLinCols * ((epi == 2 || !bf16) ? 4 : es) + 16;
  const int chunks = (K + kch - 1) / kch;
  auto lds_for = [&](int ct_per) {
    const int nbuf = ct_per * chunks > 1 ? 2 : 1;   // W staging buffers
    return (size_t)nbuf * kLinCols * (K < kch ? K : kch) * es + (size_t)kWaves * 32 * orb;
  };
  // How many workgroups share a row tile's feature tiles (col_groups, each
  // taking ct_per of them).  Cost model: the launch takes ceil(workgroups /
  // resident) generations, each as long as a workgroup's ct_per tiles plus a
  // fixed part (staging X, the first W block, the launch) worth phi tiles:
  // 1 for the plain and residual epilogues, 0.25 with GELU, whose arithmetic
  // makes a tile longer (0.5 kept the 56 x 56 x 64 fc1 at one workgroup a
  // row tile: 50.7 us against 47.8 with three).  Resident workgroups come from the kernel's
  // occupancy at each choice's LDS (one W buffer when a workgroup has one
  // step).  On MI355X this picks the measured best split (or one within 1
  // us of it) on every stage shape whose K fits one chunk (e.g. the 14 x 14
  // x 256 fc1: 42 -> 28 us against the fixed target it replaced).
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // the largest choice's LDS (two W buffers whenever a workgroup has more
  // than one step) bounds them all
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds_for(a.col_tiles));
  if (e != hipSuccess) return e;
  const double phi = epi == 1 ? 0.25 : 1.0;
  double best = 0.0;
  int best_cg = 1;
  // (measured with K in one chunk; with several chunks, as in fc2, the
  // earlier rule stays: about 512 workgroups, feature tiles shared only when
  // there are fewer row tiles)
  if (chunks > 1) {
    int cg = (512 + a.row_tiles - 1) / a.row_tiles;
    cg = cg < 1 ? 1 : cg > a.col_tiles ? a.col_tiles : cg;
    const int per = (a.col_tiles + cg - 1) / cg;
    best_cg = (a.col_tiles + per - 1) / per;            // no empty group
    best = 1.0;
  }
  for (int ct_per = a.col_tiles; ct_per >= 1 && chunks == 1; --ct_per) {
    const int cg = (a.col_tiles + ct_per - 1) / ct_per;
    if ((a.col_tiles + cg - 1) / cg != ct_per) continue;      // same split as a larger ct_per
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds_for(ct_per));
    if (e != hipSuccess) return e;
    if (per_cu < 1) continue;
    const long long wgs = (long long)a.row_tiles * cg, res = (long long)per_cu * cus;
    const double cost = (double)((wgs + res - 1) / res) * (ct_per + phi);
    if (best == 0.0 || cost < best) { best = cost; best_cg = cg; }
  }
  if (best == 0.0) return hipErrorInvalidConfiguration;
  a.col_groups = best_cg;
  a.per_xcd = (a.row_tiles * a.col_groups + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(a.per_xcd * kXcds));
  const int ct_per = (a.col_tiles + a.col_groups - 1) / a.col_groups;
  a.nbuf = ct_per * chunks > 1 ? 2 : 1;   // steps of a workgroup
  const size_t lds = lds_for(ct_per);
#define BRA_LIN(BB, KK, EE) \
  hipLaunchKernelGGL((linear_kernel<BB, KK, EE>), grid, dim3(kThreads), lds, st, a)
#define BRA_LIN_E(BB, KK) \
  if (epi == 0) BRA_LIN(BB, KK, 0); else if (epi == 1) BRA_LIN(BB, KK, 1); else BRA_LIN(BB, KK, 2)
  if (bf16 && kch == 64) { BRA_LIN_E(true, 64); }
  else if (bf16 && kch == 128) { BRA_LIN_E(true, 128); }
  else if (bf16) { BRA_LIN_E(true, 256); }
  else { BRA_LIN_E(false, 64); }
#undef BRA_LIN_E
#undef BRA_LIN
  return hipGetLastError();
}

hipError_t launch_means_proj(const double* xm, int rows, int C, const void* w_qkv,
                             const float* b_qkv, bool bf16, double* qm, double* km,
                             hipStream_t st) {
  if (rows <= 0 || C <= 0 || C % 32) return hipErrorInvalidValue;
  MeansArgs a;
  a.xm = xm; a.w = w_qkv; a.b = b_qkv; a.qm = qm; a.km = km;
  a.rows = rows; a.C = C;
  a.col_tiles = 2 * C / 16;
  const int nt = C <= 64 ? 1 : 2;                  // column tiles a wavefront
  a.col_blocks = (a.col_tiles + nt * kWaves - 1) / (nt * kWaves);
  const dim3 grid((unsigned)(((rows + 15) / 16) * a.col_blocks));
#define BRA_MP(BB, NN) hipLaunchKernelGGL((means_proj_kernel<BB, NN, 8>), grid, dim3(kThreads), 0, st, a)
  if (bf16) {
    if (nt == 1) BRA_MP(true, 1); else BRA_MP(true, 2);
  } else {
    if (nt == 1) BRA_MP(false, 1); else BRA_MP(false, 2);
  }
#undef BRA_MP
  return hipGetLastError();
}

}  // namespace bra
