// Backward pass of the BRA forward with the routing index held fixed
// (gfx950, bf16 inputs, head width 32).
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3 forward steps; §5 training with the routing kept fixed), p2 =
// snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的计算
// 范式" (§4 TopkRouting detaches its inputs unless diff_routing is set; the
// LePE depthwise Conv2d; §5 a fixed routing index).
//
// With p = softmax(s), s = scale q k^T over the routed keys of a query
// region, and do the output gradient: dv = p^T do, dp = do v^T,
// ds = p (dp - D) with D = rowsum(p dp) = do . o, dq = scale ds k,
// dk = scale ds^T q.  Two kernels, no atomics, a fixed order of every sum:
//   bwd_dq_kernel   per (image, query region, head): all routed keys in
//                   LDS, 16 queries per wavefront; s and dp on the matrix
//                   cores, the softmax in float32, dq = scale K^T ds^T with
//                   ds split into hi + lo bf16 operands;
//                   writes dq and each query's log2-sum-exp and D;
//   bwd_dkv_kernel  per (image, key region, head): 16 keys per wavefront
//                   held as operands; walks the query regions that route to
//                   the key region (an inverse routing list in ascending
//                   order), recomputes p from the saved log-sum-exp and
//                   accumulates dv^T = do^T p and dk^T = q^T ds in
//                   registers (p and ds as hi + lo bf16 operands); adds the
//                   LePE term of dV before its single rounding.
// The LePE gradient: dV_L is the transposed depthwise conv of dout (float32,
// consumed by bwd_dkv_kernel); dw and db are sums over the pixels, per image
// row first, then over the rows.

#include "device_common.h"

namespace bra {
namespace {

constexpr int kHd = 32;                 // head width
constexpr int kBwMaxKeys = 256;         // routed keys held in LDS by bwd_dq_kernel
constexpr uint32_t kBwOob = 0x80000000u;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane row, lane j
// receives element j % 4 of the four 16-bit elements addressed by lanes
// j / 4 + 4e, e = 0..3 (as element e).
__device__ __forceinline__ uint2 tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A [row][32 channel] bf16 tile, 64 bytes a row, 16-byte chunk c of row r
// at chunk c ^ ((r >> 2) & 3): the 16 rows an operand read touches fall in
// distinct bank groups, and so do the rows of a transposing read.
__device__ __forceinline__ int tswz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ uint16_t* trow(uint16_t* t, int r, int c) {
  return t + r * kHd + ((c ^ tswz(r)) << 3);
}

// Operand (16 rows x 32 channels) of row block rb: lane (lq, lg) gets row
// 16 rb + lq, channels 8 lg .. 8 lg + 7.
__device__ __forceinline__ bf16x8 row_op(const uint16_t* t, int r, int lg) {
  return *(const bf16x8*)(t + r * kHd + ((lg ^ tswz(r)) << 3));
}

// Transposed operands of the 32 rows 32 h .. 32 h + 31 of a tile, in the
// slot order of a packed 16-row pair (slots e < 4: rows 32h + 4lg + e, e >= 4:
// 32h + 16 + 4lg + e - 4): lane (lq, lg) gets channel lq (first) or 16 + lq
// (second) of those rows.
__device__ __forceinline__ void trans_ops(const uint16_t* t, int h, int lq, int lg, bf16x8& lo,
                                          bf16x8& hi) {
  const int vrow = 4 * lg + (lq >> 2);
  const int sw = tswz(vrow);                       // the same for vrow + 16m
  const uint16_t* base = t + (32 * h + vrow) * kHd + 4 * (lq & 1);
  const int ca = (((lq >> 1) & 1) ^ sw) * 8;       // channels 0 .. 15
  const int cb = ((2 + ((lq >> 1) & 1)) ^ sw) * 8; // channels 16 .. 31
  const uint2 a0 = tr16(base + ca), a1 = tr16(base + 16 * kHd + ca);
  const uint2 c0 = tr16(base + cb), c1 = tr16(base + 16 * kHd + cb);
  lo = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
  hi = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
}

// Two floats as hi + lo bf16 pairs (lo = the rounded remainder): 16
// significant bits through a bf16 matrix product, at twice the products.
// The gradient products take p and ds this way: a bf16 operand alone costs
// half an ulp of bf16 on the dominant terms of a peaked softmax.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}

struct BwArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const int32_t* idx;     // [B, R, topk]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* lse;             // [B, H, W, heads]: log2-sum-exp of the scaled logits
  float* dd;              // [B, H, W, heads]: D = rowsum(p dp)
  const float* dv_lepe;   // [B, H, W, C] float32 or null
  const int32_t* inv_off; // [B, R + 1] offsets into inv_rows
  const int32_t* inv_rows;// [B, R * topk] query regions routing to each key region
  int B, H, W, C, S, R, hs, ws, n, heads, topk;
  float scale, scale_log2;
};

// element offset of token t of region r (image-relative)
__device__ __forceinline__ int tok_off(const BwArgs& a, int r, int t) {
  const int ry = r / a.S, rx = r - ry * a.S;
  const int ty = t / a.ws, tx = t - ty * a.ws;
  return ((ry * a.hs + ty) * a.W + rx * a.ws + tx) * a.C;
}

template <int NH>                        // 32-key steps: KC rounded up to 32 * NH
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Ks = (uint16_t*)lds;
  constexpr int KCP = 32 * NH;
  const int KC = a.topk * a.n;
  uint16_t* Vs = Ks + KCP * kHd;
  const int u = blockIdx.x;
  const int h = u % a.heads, br = u / a.heads;
  const int b = br / a.R, r = br - b * a.R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 15, lg = lane >> 4;
  const uint32_t img = (uint32_t)a.H * a.W * a.C;
  const auto Kr = rsrc(a.k + (size_t)b * img, img * 2), Vr = rsrc(a.v + (size_t)b * img, img * 2);
  const auto Qr = rsrc(a.q + (size_t)b * img, img * 2), Gr = rsrc(a.dout + (size_t)b * img, img * 2);
  const int32_t* route = a.idx + (size_t)br * a.topk;
  // routed keys (regions in route order, tokens row-major), zero past KC
  for (int e = tid; e < KCP * 4; e += kThreads) {
    const int kk = e >> 2, c = e & 3;
    uint32_t off = kBwOob;
    if (kk < KC) {
      const int reg = min(max(route[kk / a.n], 0), a.R - 1);
      off = (tok_off(a, reg, kk % a.n) + h * kHd + 8 * c) * 2;
    }
    *(uint4*)trow(Ks, kk, c) = ld16(Kr, off);
    *(uint4*)trow(Vs, kk, c) = ld16(Vr, off);
  }
  __syncthreads();
  const float c2 = a.scale_log2;
  const int nqb = (a.n + 15) / 16;
  for (int qb = wave; qb < nqb; qb += kWaves) {
    const int q = 16 * qb + lq;
    const bool qok = q < a.n;
    const uint32_t qoff = qok ? (tok_off(a, r, q) + h * kHd + 8 * lg) * 2 : kBwOob;
    const bf16x8 qop = __builtin_bit_cast(bf16x8, ld16(Qr, qoff));
    const bf16x8 gop = __builtin_bit_cast(bf16x8, ld16(Gr, qoff));
    // s^T and dp^T: lane holds keys 16 kb + 4 lg + e of query lq
    float s[KCP / 4], dp[KCP / 4];
    float m = -3.0e38f;
#pragma unroll
    for (int kb = 0; kb < KCP / 16; ++kb) {
      const int key = 16 * kb + lq;
      const f32x4 sv = mfma16(row_op(Ks, key, lg), qop, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 pv = mfma16(row_op(Vs, key, lg), gop, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool kok = 16 * kb + 4 * lg + e < KC;
        s[4 * kb + e] = kok ? sv[e] : -3.0e38f;
        dp[4 * kb + e] = pv[e];
        m = fmaxf(m, s[4 * kb + e]);
      }
    }
    m = fmaxf(m, xor16(m));
    m = fmaxf(m, xor32(m));
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < KCP / 4; ++e) {
      s[e] = __builtin_amdgcn_exp2f((s[e] - m) * c2);   // p, unnormalised (0 past KC)
      l += s[e];
    }
    l += xor16(l);
    l += xor32(l);
    const float inv = 1.0f / l;
    float D = 0.f;
#pragma unroll
    for (int e = 0; e < KCP / 4; ++e) D = fmaf(s[e] * inv, dp[e], D);
    D += xor16(D);
    D += xor32(D);
    // ds^T packed in the slot order of 32-key steps, then dq^T = K^T ds^T
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      uint32_t pk[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // s[4 kb + e] holds key 16 kb + 4 lg + e: slots of step hh are
        // s[8 hh .. 8 hh + 7] (kb = 2 hh, then 2 hh + 1)
        const int e0 = 8 * hh + 2 * j;
        split_bf16x2(s[e0] * inv * (dp[e0] - D), s[e0 + 1] * inv * (dp[e0 + 1] - D), pk[j], pl[j]);
      }
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      const bf16x8 dsl = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
      bf16x8 klo, khi;
      trans_ops(Ks, hh, lq, lg, klo, khi);
      acc0 = mfma16(klo, dsb, acc0);
      acc1 = mfma16(khi, dsb, acc1);
      acc0 = mfma16(klo, dsl, acc0);
      acc1 = mfma16(khi, dsl, acc1);
    }
    if (qok) {
      // lane holds channels 4 lg + e (acc0) and 16 + 4 lg + e (acc1) of query q
      uint16_t* dqp = a.dq + (size_t)b * img + tok_off(a, r, q) + h * kHd;
      *(uint2*)(dqp + 4 * lg) = make_uint2(pack_bf16x2(acc0[0] * a.scale, acc0[1] * a.scale),
                                           pack_bf16x2(acc0[2] * a.scale, acc0[3] * a.scale));
      *(uint2*)(dqp + 16 + 4 * lg) = make_uint2(pack_bf16x2(acc1[0] * a.scale, acc1[1] * a.scale),
                                                pack_bf16x2(acc1[2] * a.scale, acc1[3] * a.scale));
      if (lg == 0) {
        const size_t pix = (size_t)b * a.H * a.W + tok_off(a, r, q) / a.C;
        a.lse[pix * a.heads + h] = m * c2 + __log2f(l);
        a.dd[pix * a.heads + h] = D;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(BwArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int NQP = (a.n + 31) / 32 * 32;
  uint16_t* Qs = (uint16_t*)lds;
  uint16_t* Gs = Qs + NQP * kHd;
  float* Ls = (float*)(Gs + NQP * kHd);            // log2-sum-exp of the staged queries
  float* Ds = Ls + NQP;
  const int u = blockIdx.x;
  const int h = u % a.heads, bs = u / a.heads;
  const int b = bs / a.R, s = bs - b * a.R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 15, lg = lane >> 4;
  const uint32_t img = (uint32_t)a.H * a.W * a.C;
  const auto Kr = rsrc(a.k + (size_t)b * img, img * 2), Vr = rsrc(a.v + (size_t)b * img, img * 2);
  const auto Qr = rsrc(a.q + (size_t)b * img, img * 2), Gr = rsrc(a.dout + (size_t)b * img, img * 2);
  const float c2 = a.scale_log2;
  const int nkb = (a.n + 15) / 16;
  const int beg = a.inv_off[b * (a.R + 1) + s], end = a.inv_off[b * (a.R + 1) + s + 1];
  const int32_t* rows = a.inv_rows + (size_t)b * a.R * a.topk;
  for (int kb = wave; kb < nkb + ((nkb + kWaves - 1) / kWaves * kWaves - nkb); kb += kWaves) {
    // every wavefront runs the same number of passes (the barriers below)
    const bool kact = kb < nkb;
    const int key = 16 * kb + lq;
    const bool kok = kact && key < a.n;
    const uint32_t koff = kok ? (tok_off(a, s, key) + h * kHd + 8 * lg) * 2 : kBwOob;
    const bf16x8 kop = __builtin_bit_cast(bf16x8, ld16(Kr, koff));
    const bf16x8 vop = __builtin_bit_cast(bf16x8, ld16(Vr, koff));
    f32x4 ak0 = {0.f, 0.f, 0.f, 0.f}, ak1 = ak0, av0 = ak0, av1 = ak0;
    for (int it = beg; it < end; ++it) {
      const int r = rows[it];
      __syncthreads();                              // the previous tiles are consumed
      for (int e = tid; e < NQP * 4; e += kThreads) {
        const int qq = e >> 2, c = e & 3;
        const uint32_t off = qq < a.n ? (tok_off(a, r, qq) + h * kHd + 8 * c) * 2 : kBwOob;
        *(uint4*)trow(Qs, qq, c) = ld16(Qr, off);
        *(uint4*)trow(Gs, qq, c) = ld16(Gr, off);
      }
      for (int qq = tid; qq < NQP; qq += kThreads) {
        float lv = 3.0e38f, dv = 0.f;               // padding queries: p = 0
        if (qq < a.n) {
          const size_t pix = (size_t)b * a.H * a.W + tok_off(a, r, qq) / a.C;
          lv = a.lse[pix * a.heads + h];
          dv = a.dd[pix * a.heads + h];
        }
        Ls[qq] = lv;
        Ds[qq] = dv;
      }
      __syncthreads();
      if (!kact) continue;
      for (int hh = 0; hh < NQP / 32; ++hh) {
        uint32_t pp[4], pd[4], ppl[4], pdl[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int qrow = 32 * hh + 16 * half + lq;  // A rows: queries
          const f32x4 sv = mfma16(row_op(Qs, qrow, lg), kop, f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 gv = mfma16(row_op(Gs, qrow, lg), vop, f32x4{0.f, 0.f, 0.f, 0.f});
          // lane holds key lq, queries 32hh + 16half + 4lg + e
          float p[4], ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qe = 32 * hh + 16 * half + 4 * lg + e;
            p[e] = __builtin_amdgcn_exp2f(sv[e] * c2 - Ls[qe]);
            ds[e] = p[e] * (gv[e] - Ds[qe]);
          }
          split_bf16x2(p[0], p[1], pp[2 * half], ppl[2 * half]);
          split_bf16x2(p[2], p[3], pp[2 * half + 1], ppl[2 * half + 1]);
          split_bf16x2(ds[0], ds[1], pd[2 * half], pdl[2 * half]);
          split_bf16x2(ds[2], ds[3], pd[2 * half + 1], pdl[2 * half + 1]);
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pp[0], pp[1], pp[2], pp[3]));
        const bf16x8 pbl = __builtin_bit_cast(bf16x8, make_uint4(ppl[0], ppl[1], ppl[2], ppl[3]));
        const bf16x8 db = __builtin_bit_cast(bf16x8, make_uint4(pd[0], pd[1], pd[2], pd[3]));
        const bf16x8 dbl = __builtin_bit_cast(bf16x8, make_uint4(pdl[0], pdl[1], pdl[2], pdl[3]));
        bf16x8 lo, hi;
        trans_ops(Gs, hh, lq, lg, lo, hi);          // dO^T
        av0 = mfma16(lo, pb, av0);
        av1 = mfma16(hi, pb, av1);
        av0 = mfma16(lo, pbl, av0);
        av1 = mfma16(hi, pbl, av1);
        trans_ops(Qs, hh, lq, lg, lo, hi);          // Q^T
        ak0 = mfma16(lo, db, ak0);
        ak1 = mfma16(hi, db, ak1);
        ak0 = mfma16(lo, dbl, ak0);
        ak1 = mfma16(hi, dbl, ak1);
      }
    }
    if (kok) {
      // lane holds channels 4 lg + e (acc 0) and 16 + 4 lg + e (acc 1) of key `key`
      const int to = tok_off(a, s, key) + h * kHd;
      float l0[4] = {0.f, 0.f, 0.f, 0.f}, l1[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.dv_lepe) {
        const float4 x0 = *(const float4*)(a.dv_lepe + (size_t)b * img + to + 4 * lg);
        const float4 x1 = *(const float4*)(a.dv_lepe + (size_t)b * img + to + 16 + 4 * lg);
        l0[0] = x0.x; l0[1] = x0.y; l0[2] = x0.z; l0[3] = x0.w;
        l1[0] = x1.x; l1[1] = x1.y; l1[2] = x1.z; l1[3] = x1.w;
      }
      uint16_t* dkp = a.dk + (size_t)b * img + to;
      uint16_t* dvp = a.dv + (size_t)b * img + to;
      const float sc = a.scale;
      *(uint2*)(dkp + 4 * lg) = make_uint2(pack_bf16x2(ak0[0] * sc, ak0[1] * sc),
                                           pack_bf16x2(ak0[2] * sc, ak0[3] * sc));
      *(uint2*)(dkp + 16 + 4 * lg) = make_uint2(pack_bf16x2(ak1[0] * sc, ak1[1] * sc),
                                                pack_bf16x2(ak1[2] * sc, ak1[3] * sc));
      *(uint2*)(dvp + 4 * lg) = make_uint2(pack_bf16x2(av0[0] + l0[0], av0[1] + l0[1]),
                                           pack_bf16x2(av0[2] + l0[2], av0[3] + l0[3]));
      *(uint2*)(dvp + 16 + 4 * lg) = make_uint2(pack_bf16x2(av1[0] + l1[0], av1[1] + l1[1]),
                                                pack_bf16x2(av1[2] + l1[2], av1[3] + l1[3]));
    }
  }
}

// Inverse routing: for image b and key region s, the query regions r with
// s in idx[b][r] (with multiplicity), ascending in r then slot.  One thread
// per (b, s) scans the image's index: deterministic, no atomics.
__global__ __launch_bounds__(kThreads) void inv_route_kernel(const int32_t* idx, int B, int R,
                                                              int topk, int32_t* off,
                                                              int32_t* rows) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= B * R) return;
  const int b = t / R, s = t - b * R;
  const int32_t* ib = idx + (size_t)b * R * topk;
  int before = 0, cnt = 0;
  for (int e = 0; e < R * topk; ++e) {
    const int reg = min(max(ib[e], 0), R - 1);
    before += reg < s;
    cnt += reg == s;
  }
  int32_t* rb = rows + (size_t)b * R * topk + before;
  int k = 0;
  for (int e = 0; e < R * topk && k < cnt; ++e) {
    const int reg = min(max(ib[e], 0), R - 1);
    if (reg == s) rb[k++] = e / topk;
  }
  off[b * (R + 1) + s] = before;
  if (s == R - 1) off[b * (R + 1) + R] = before + cnt;
}

// dV_L[y, x, c] = sum_{i,j} w[c, i, j] dout[y - i + P, x - j + P, c] (zero
// outside), float32.  Thread (x, g) of one image row: 16-byte channel group
// g of pixel x; the block's weights are staged in LDS as [tap][channel].
template <int KS>
__global__ __launch_bounds__(kThreads) void lepe_dv_kernel(const uint16_t* g, const float* w,
                                                           int H, int W, int C, float* dvl) {
  extern __shared__ float wt[];                     // [KS * KS][C]
  constexpr int P = KS / 2, KK = KS * KS;
  for (int e = threadIdx.x; e < KK * C; e += kThreads) {
    const int c = e / KK, t = e - c * KK;
    wt[t * C + c] = w[e];
  }
  __syncthreads();
  const int G = C / 8;
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= W * G) return;
  const int y = blockIdx.y, b = blockIdx.z;
  const int x = t / G, gi = t - x * G;
  const uint16_t* gb = g + (size_t)b * H * W * C;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < KS; ++i) {
    const int yy = y - i + P;
    if ((unsigned)yy >= (unsigned)H) continue;
    for (int j = 0; j < KS; ++j) {
      const int xx = x - j + P;
      if ((unsigned)xx >= (unsigned)W) continue;
      float v[8];
      unpack16<true>(*(const uint4*)(gb + ((size_t)yy * W + xx) * C + gi * 8), v);
      const float4 w0 = *(const float4*)(wt + (i * KS + j) * C + gi * 8);
      const float4 w1 = *(const float4*)(wt + (i * KS + j) * C + gi * 8 + 4);
      acc[0] = fmaf(w0.x, v[0], acc[0]); acc[1] = fmaf(w0.y, v[1], acc[1]);
      acc[2] = fmaf(w0.z, v[2], acc[2]); acc[3] = fmaf(w0.w, v[3], acc[3]);
      acc[4] = fmaf(w1.x, v[4], acc[4]); acc[5] = fmaf(w1.y, v[5], acc[5]);
      acc[6] = fmaf(w1.z, v[6], acc[6]); acc[7] = fmaf(w1.w, v[7], acc[7]);
    }
  }
  float* o = dvl + (((size_t)b * H + y) * W + x) * C + gi * 8;
  *(float4*)o = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *(float4*)(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Per-row partial sums of dw and db: one workgroup per (image, row), a
// thread per channel (consecutive threads read consecutive channels of a
// pixel, so the loads coalesce); each thread walks the row's pixels and the
// taps in order.  part[(b * H + y) * C + c][KK + 1]: the KK taps, then db.
template <int KS>
__global__ __launch_bounds__(kThreads) void lepe_dw_rows_kernel(const uint16_t* g,
                                                                const uint16_t* v, int H, int W,
                                                                int C, float* part) {
  constexpr int P = KS / 2, KK = KS * KS;
  const int y = blockIdx.y, b = blockIdx.z;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  const uint16_t* gb = g + (size_t)b * H * W * C + c;
  const uint16_t* vb = v + (size_t)b * H * W * C + c;
  float acc[KK + 1];
#pragma unroll
  for (int t = 0; t <= KK; ++t) acc[t] = 0.f;
  for (int x = 0; x < W; ++x) {
    const float gv = __uint_as_float((uint32_t)gb[((size_t)y * W + x) * C] << 16);
    acc[KK] += gv;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int yy = y + i - P;
      if ((unsigned)yy >= (unsigned)H) continue;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int xx = x + j - P;
        if ((unsigned)xx >= (unsigned)W) continue;
        const float vv = __uint_as_float((uint32_t)vb[((size_t)yy * W + xx) * C] << 16);
        acc[i * KS + j] = fmaf(gv, vv, acc[i * KS + j]);
      }
    }
  }
  float* pp = part + (((size_t)b * H + y) * C + c) * (KK + 1);
#pragma unroll
  for (int t = 0; t <= KK; ++t) pp[t] = acc[t];
}

// dw[c][t] and db[c]: the sums of the per-row partials over all rows, one
// thread per (c, t), rows in order.
__global__ __launch_bounds__(kThreads) void lepe_dw_sum_kernel(const float* part, int rows, int C,
                                                               int KK, float* dw, float* db) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= C * (KK + 1)) return;
  const int c = e / (KK + 1), t = e - c * (KK + 1);
  double s = 0.0;                                   // many rows: keep the sum exact enough
  for (int r = 0; r < rows; ++r) s += part[((size_t)r * C + c) * (KK + 1) + t];
  if (t < KK) dw[c * KK + t] = (float)s;
  else if (db) db[c] = (float)s;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk, int ks,
                           bool lepe) {
  const size_t px = (size_t)B * H * W;
  size_t bytes = 2 * px * heads * sizeof(float);                   // lse, D
  bytes += ((size_t)B * (S * S + 1) + (size_t)B * S * S * topk) * sizeof(int32_t);
  bytes = (bytes + 255) / 256 * 256;
  if (lepe) {
    bytes += px * C * sizeof(float);                               // dV_L
    bytes += (size_t)B * H * C * (ks * ks + 1) * sizeof(float);    // per-row partials
  }
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* dout, const Shape& s, float attn_scale, const float* w,
                           int ks, void* dq, void* dk, void* dvv, float* dw, float* db, void* ws,
                           hipStream_t st) {
  if (s.C != s.heads * kHd || s.topk * s.n > kBwMaxKeys) return hipErrorNotSupported;
  // buffer offsets of one image (bytes) stay below 2^31
  if ((long long)s.H * s.W * s.C * 2 >= (long long)kBwOob) return hipErrorNotSupported;
  BwArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout; a.idx = idx;
  a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dvv;
  a.B = s.B; a.H = s.H; a.W = s.W; a.C = s.C; a.S = s.S; a.R = s.R; a.hs = s.hs; a.ws = s.ws;
  a.n = s.n; a.heads = s.heads; a.topk = s.topk;
  a.scale = attn_scale;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  const size_t px = (size_t)s.B * s.H * s.W;
  unsigned char* w8 = (unsigned char*)ws;
  a.lse = (float*)w8;
  a.dd = a.lse + px * s.heads;
  a.inv_off = (const int32_t*)(a.dd + px * s.heads);
  int32_t* inv_off = (int32_t*)a.inv_off;
  int32_t* inv_rows = inv_off + (size_t)s.B * (s.R + 1);
  a.inv_rows = inv_rows;
  size_t used = 2 * px * s.heads * sizeof(float) +
                ((size_t)s.B * (s.R + 1) + (size_t)s.B * s.R * s.topk) * sizeof(int32_t);
  used = (used + 255) / 256 * 256;
  float* dvl = w ? (float*)(w8 + used) : nullptr;
  float* part = w ? dvl + px * s.C : nullptr;
  a.dv_lepe = dvl;
  hipError_t e;
  // inverse routing lists
  hipLaunchKernelGGL(inv_route_kernel, dim3((unsigned)((s.B * s.R + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, idx, s.B, s.R, s.topk, inv_off, inv_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // LePE: dV_L, dw, db
  if (w) {
    if (s.H > 65535 || s.B > 65535 || s.C > 65535) return hipErrorNotSupported;
    const dim3 g1((unsigned)((s.W * (s.C / 8) + kThreads - 1) / kThreads), (unsigned)s.H, (unsigned)s.B);
    const size_t wl = (size_t)ks * ks * s.C * sizeof(float);
    const int tpb = s.C < kThreads ? s.C : kThreads;
    const dim3 g2((unsigned)((s.C + tpb - 1) / tpb), (unsigned)s.H, (unsigned)s.B);
    const int rows = s.B * s.H, KK = ks * ks;
    const dim3 g3((unsigned)((s.C * (KK + 1) + kThreads - 1) / kThreads));
#define BRA_LEPE_BW(KSV)                                                                       \
    case KSV: {                                                                                \
      e = hipFuncSetAttribute((const void*)lepe_dv_kernel<KSV>,                                \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)wl);            \
      if (e != hipSuccess) return e;                                                           \
      hipLaunchKernelGGL(lepe_dv_kernel<KSV>, g1, dim3(kThreads), wl, st, (const uint16_t*)dout, \
                         w, s.H, s.W, s.C, dvl);                                               \
      hipLaunchKernelGGL(lepe_dw_rows_kernel<KSV>, g2, dim3(tpb), 0, st,                       \
                         (const uint16_t*)dout, (const uint16_t*)v, s.H, s.W, s.C, part);      \
      break;                                                                                   \
    }
    switch (ks) {
      BRA_LEPE_BW(1) BRA_LEPE_BW(3) BRA_LEPE_BW(5) BRA_LEPE_BW(7)
      default: return hipErrorInvalidValue;
    }
#undef BRA_LEPE_BW
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(lepe_dw_sum_kernel, g3, dim3(kThreads), 0, st, part, rows, s.C, KK, dw, db);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dq (and the saved statistics), then dk / dv
  const int NH = (s.topk * s.n + 31) / 32;
  const size_t lq = (size_t)2 * 32 * NH * kHd * 2;
  const unsigned units = (unsigned)(s.B * s.R * s.heads);
#define BRA_DQ(NN)                                                                             \
    case NN:                                                                                   \
      e = hipFuncSetAttribute((const void*)bwd_dq_kernel<NN>,                                  \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lq);            \
      if (e != hipSuccess) return e;                                                           \
      hipLaunchKernelGGL(bwd_dq_kernel<NN>, dim3(units), dim3(kThreads), lq, st, a);           \
      break;
  switch (NH) {
    BRA_DQ(1) BRA_DQ(2) BRA_DQ(3) BRA_DQ(4) BRA_DQ(5) BRA_DQ(6) BRA_DQ(7) BRA_DQ(8)
    default: return hipErrorNotSupported;
  }
#undef BRA_DQ
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NQP = (s.n + 31) / 32 * 32;
  const size_t lk = (size_t)2 * NQP * kHd * 2 + (size_t)2 * NQP * sizeof(float);
  e = hipFuncSetAttribute((const void*)bwd_dkv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lk);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3(units), dim3(kThreads), lk, st, a);
  return hipGetLastError();
}

}  // namespace bra
