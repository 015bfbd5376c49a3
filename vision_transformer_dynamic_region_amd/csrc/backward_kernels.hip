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
//                   cores, the softmax in float32 (two sweeps), dq = scale
//                   K^T ds^T with ds split into hi + lo bf16 operands;
//                   writes dq and each query's log2-sum-exp and D;
//   bwd_dkv_kernel  per (image, key region, head): 16 keys per wavefront
//                   held as operands; walks the query regions that route to
//                   the key region (an inverse routing list in ascending
//                   order), recomputes p from the saved log-sum-exp and
//                   accumulates dv^T = do^T p and dk^T = q^T ds in
//                   registers (p and ds as hi + lo bf16 operands); adds the
//                   LePE term of dV (the transposed depthwise conv of dout)
//                   before its single rounding.
// dw and db are sums over the pixels: float32 partial sums per workgroup
// (a strip of rows of a few columns), then float64 sums of the partials.

#include "device_common.h"
#include "launch_plan.h"

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
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
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
  const float* dv_lepe;   // [B, H, W, C] float32: the LePE term of dV, or null
  int B, H, W, C, S, R, hs, ws, n, heads, topk;
  float scale, scale_log2;
  FastDiv f_S, f_ws, f_n, f_topk, f_R;   // divisions by launch constants (no integer divide)
};

// pixel index and element offset of token t of region r (image-relative)
__device__ __forceinline__ int tok_pix(const BwArgs& a, int r, int t) {
  const int ry = fdiv(r, a.f_S), rx = r - ry * a.S;
  const int ty = fdiv(t, a.f_ws), tx = t - ty * a.ws;
  return (ry * a.hs + ty) * a.W + rx * a.ws + tx;
}
__device__ __forceinline__ int tok_off(const BwArgs& a, int r, int t) {
  return tok_pix(a, r, t) * a.C;
}

// Query-centric pass, two sweeps over the routed keys held in LDS: the
// first keeps a running maximum, sum of exponentials and sum of p * dp per
// lane (each lane sees a quarter of a query's keys) and combines the four
// lanes of a query at the end, giving its log-sum-exp and D; the second
// recomputes s and dp, forms ds = p (dp - D) and accumulates dq^T = K^T ds^T.
// Nothing is held per key, so the register count does not grow with topk * n.
template <bool FULL>                     // FULL: topk * n is a multiple of 32, no key is masked
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwArgs a, int NH, int hpw) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int KCP = 32 * NH;
  const int KC = a.topk * a.n;
  uint16_t* Ks0 = (uint16_t*)lds;                  // [hpw][KCP][32]
  uint16_t* Vs0 = Ks0 + hpw * KCP * kHd;           // [hpw][KCP][32]
  const int ng = a.heads / hpw;
  const int u = blockIdx.x;
  const int hg = u % ng, br = u / ng;
  const int b = fdiv(br, a.f_R), r = br - b * a.R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 15, lg = lane >> 4;
  const int lh = hpw == 4 ? 2 : hpw == 2 ? 1 : 0;   // log2(hpw)
  const uint32_t img = (uint32_t)a.H * a.W * a.C;
  const auto Kr = rsrc(a.k + (size_t)b * img, img * 2), Vr = rsrc(a.v + (size_t)b * img, img * 2);
  const auto Qr = rsrc(a.q + (size_t)b * img, img * 2), Gr = rsrc(a.dout + (size_t)b * img, img * 2);
  const int32_t* route = a.idx + (size_t)br * a.topk;
  const int nqb = (a.n + 15) / 16;
  const int ntask = nqb * hpw;                     // (query block, head) pairs
  auto qoff_of = [&](int t) -> uint32_t {
    const int qb = t >> lh, hh = hg * hpw + (t & (hpw - 1));
    const int q = 16 * qb + lq;
    return (t < ntask && q < a.n) ? (tok_off(a, r, q) + hh * kHd + 8 * lg) * 2 : kBwOob;
  };
  // the first task's query operands are in flight during the staging
  uint32_t qoff = qoff_of(wave);
  uint4 qn = ld16(Qr, qoff), gn = ld16(Gr, qoff);
  // routed keys of the group's heads (regions in route order, tokens
  // row-major), zero past KC; consecutive threads take consecutive 16-byte
  // chunks of a key row across the heads
  for (int e = tid; e < KCP * 4 * hpw; e += kThreads) {
    const int c = e & 3, rest = e >> 2, kk = rest >> lh, hl = rest & (hpw - 1);
    uint32_t off = kBwOob;
    if (kk < KC) {
      const int j = fdiv(kk, a.f_n);
      const int reg = min(max(route[j], 0), a.R - 1);
      off = (tok_off(a, reg, kk - j * a.n) + (hg * hpw + hl) * kHd + 8 * c) * 2;
    }
    *(uint4*)trow(Ks0 + hl * KCP * kHd, kk, c) = ld16(Kr, off);
    *(uint4*)trow(Vs0 + hl * KCP * kHd, kk, c) = ld16(Vr, off);
  }
  __syncthreads();
  const float c2 = a.scale_log2;
  for (int t = wave; t < ntask; t += kWaves) {
    const int qb = t >> lh, hl = t & (hpw - 1), h = hg * hpw + hl;
    const uint16_t* Ks = Ks0 + hl * KCP * kHd;
    const uint16_t* Vs = Vs0 + hl * KCP * kHd;
    const int q = 16 * qb + lq;
    const bool qok = q < a.n;
    const bf16x8 qop = __builtin_bit_cast(bf16x8, qn);
    const bf16x8 gop = __builtin_bit_cast(bf16x8, gn);
    qoff = qoff_of(t + kWaves);
    qn = ld16(Qr, qoff);
    gn = ld16(Gr, qoff);
    // sweep 1: lane-local running max m, sum l of 2^((s - m) c2), sum D of
    // those weights times dp (keys 32 hh + 16 half + 4 lg + e of query lq)
    float m = -3.0e38f, l = 0.f, D = 0.f;
    for (int hh = 0; hh < NH; ++hh) {
      float sv[8], pv[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = 32 * hh + 16 * half + lq;
        const f32x4 s4 = mfma16(row_op(Ks, key, lg), qop, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 p4 = mfma16(row_op(Vs, key, lg), gop, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kok = FULL || 32 * hh + 16 * half + 4 * lg + e < KC;
          sv[4 * half + e] = kok ? s4[e] : -3.0e38f;
          pv[4 * half + e] = p4[e];
        }
      }
      float mc = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mc = fmaxf(mc, sv[e]);
      const float mn = fmaxf(m, mc);
      const float sc = __builtin_amdgcn_exp2f((m - mn) * c2);
      l *= sc;
      D *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ex = __builtin_amdgcn_exp2f((sv[e] - mn) * c2);
        const float pe = FULL || sv[e] > -1.0e38f ? ex : 0.f;
        l += pe;
        D = fmaf(pe, pv[e], D);
      }
      m = mn;
    }
    // combine the four lanes of query lq
    float mt = fmaxf(m, xor16(m));
    mt = fmaxf(mt, xor32(mt));
    const float f = __builtin_amdgcn_exp2f((m - mt) * c2);
    l *= f;
    D *= f;
    l += xor16(l);
    l += xor32(l);
    D += xor16(D);
    D += xor32(D);
    D /= l;
    const float lse = mt * c2 + __log2f(l);
    // sweep 2: ds = p (dp - D) in the slot order of each 32-key step, then
    // dq^T = K^T ds^T with ds as hi + lo bf16 operands
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int hh = 0; hh < NH; ++hh) {
      uint32_t pk[4], pl[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = 32 * hh + 16 * half + lq;
        const f32x4 s4 = mfma16(row_op(Ks, key, lg), qop, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 p4 = mfma16(row_op(Vs, key, lg), gop, f32x4{0.f, 0.f, 0.f, 0.f});
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kok = FULL || 32 * hh + 16 * half + 4 * lg + e < KC;
          const float ex = __builtin_amdgcn_exp2f(s4[e] * c2 - lse);
          const float p = kok ? ex : 0.f;
          ds[e] = p * (p4[e] - D);
        }
        split_bf16x2(ds[0], ds[1], pk[2 * half], pl[2 * half]);
        split_bf16x2(ds[2], ds[3], pk[2 * half + 1], pl[2 * half + 1]);
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
      const int qpix = tok_pix(a, r, q);
      uint16_t* dqp = a.dq + (size_t)b * img + qpix * a.C + h * kHd;
      *(uint2*)(dqp + 4 * lg) = make_uint2(pack_bf16x2(acc0[0] * a.scale, acc0[1] * a.scale),
                                           pack_bf16x2(acc0[2] * a.scale, acc0[3] * a.scale));
      *(uint2*)(dqp + 16 + 4 * lg) = make_uint2(pack_bf16x2(acc1[0] * a.scale, acc1[1] * a.scale),
                                                pack_bf16x2(acc1[2] * a.scale, acc1[3] * a.scale));
      if (lg == 0) {
        const size_t pix = (size_t)b * a.H * a.W + qpix;
        a.lse[pix * a.heads + h] = lse;
        a.dd[pix * a.heads + h] = D;
      }
    }
  }
}

// Key-centric pass.  The query regions that route to key region s are found
// by a stable compaction of the image's routing index (a ballot and a prefix
// count per wavefront, chunk after chunk, so the list is in ascending order
// of query region and slot, with repeats kept) and their query tokens are
// staged as one flat list, kDkvTile rows a tile, whatever the region size.
// Wavefronts take 16-key blocks; when a region has fewer than four blocks,
// the spare wavefronts take every QS-th 32-query sub-tile of the same key
// block (query splits), and the splits' sums are added in a fixed order at
// the end.  The LePE term of dV comes in as float32 (lepe_bwd_kernel) and is
// added before the single rounding.
constexpr int kDkvTile = 128;            // query rows staged per tile
constexpr int kDkvList = 1024;           // query regions held at once
static_assert(kDkvTile * 4 == 2 * kThreads && kDkvTile <= kThreads,
              "tile staging: two 16-byte chunks and at most one statistic a thread");

__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(BwArgs a, int hpw) {
  __shared__ __align__(16) uint16_t tiles[2 * kDkvTile * kHd];   // Q, dO tiles: [hpw][TR][32] each
  __shared__ float Ls0[kDkvTile], Ds0[kDkvTile];                  // [hpw][TR]
  __shared__ int mlist[kDkvList];
  __shared__ int wcnt[kWaves];
  const int TR = kDkvTile / hpw;                  // query rows a tile
  const int ng = a.heads / hpw;
  const int u = blockIdx.x;
  const int hg = u % ng, bs = u / ng;
  const int b = fdiv(bs, a.f_R), s = bs - b * a.R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 15, lg = lane >> 4;
  const int lh = hpw == 4 ? 2 : hpw == 2 ? 1 : 0;   // log2(hpw)
  const uint32_t img = (uint32_t)a.H * a.W * a.C;
  const auto Kr = rsrc(a.k + (size_t)b * img, img * 2), Vr = rsrc(a.v + (size_t)b * img, img * 2);
  const auto Qr = rsrc(a.q + (size_t)b * img, img * 2), Gr = rsrc(a.dout + (size_t)b * img, img * 2);
  const float c2 = a.scale_log2;
  const int RT = a.R * a.topk;
  const int32_t* ib = a.idx + (size_t)b * RT;
  const int KB = (a.n + 15) / 16;
  // roles: (head, key block) pairs, hpw * KB <= kWaves when hpw > 1; spare
  // wavefronts split the query sub-tiles (QS); with KB >= kWaves, groups of
  // kWaves key blocks one after another
  const int roles = KB >= kWaves ? kWaves : KB * hpw;
  const int QS = KB >= kWaves ? 1 : kWaves / roles;
  const int groups = KB >= kWaves ? (KB + kWaves - 1) / kWaves : 1;
  for (int grp = 0; grp < groups; ++grp) {
    const int role = wave % roles;
    const int hl = KB >= kWaves ? 0 : role / KB;
    const int kb = KB >= kWaves ? grp * kWaves + wave : role - hl * KB;
    const int split = wave / roles;
    const bool act = kb < KB && split < QS;
    const int h = hg * hpw + hl;
    uint16_t* Qs = tiles + hl * TR * kHd;
    uint16_t* Gs = tiles + kDkvTile * kHd + hl * TR * kHd;
    const float* Ls = Ls0 + hl * TR;
    const float* Ds = Ds0 + hl * TR;
    const int key = 16 * kb + lq;
    const bool kok = act && key < a.n;
    const uint32_t koff = kok ? (tok_off(a, s, key) + h * kHd + 8 * lg) * 2 : kBwOob;
    const bf16x8 kop = __builtin_bit_cast(bf16x8, ld16(Kr, koff));
    const bf16x8 vop = __builtin_bit_cast(bf16x8, ld16(Vr, koff));
    f32x4 ak0 = {0.f, 0.f, 0.f, 0.f}, ak1 = ak0, av0 = ak0, av1 = ak0;
    int e0 = 0;
    do {
      // compact the query regions routing to s, up to kDkvList of them
      int cnt = 0;
      while (e0 < RT && cnt <= kDkvList - kThreads) {
        const int e = e0 + tid;
        const bool pred = e < RT && min(max(ib[e], 0), a.R - 1) == s;
        const uint64_t bal = __ballot(pred);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0) wcnt[wave] = __popcll(bal);
        __syncthreads();
        int base = cnt, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const int c = wcnt[w];
          base += w < wave ? c : 0;
          tot += c;
        }
        if (pred) mlist[base + below] = fdiv(e, a.f_topk);
        cnt += tot;
        e0 += kThreads;
        __syncthreads();
      }
      const int nrows = cnt * a.n;
      for (int t0 = 0; t0 < nrows; t0 += TR) {
        // consecutive threads take consecutive 16-byte chunks of a query row
        // across the group's heads (two chunks a thread); every load of the
        // tile, the statistics included, is issued before the first LDS store
        uint4 fq[2], fg[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = tid + kThreads * u;
          const int c = e & 3, rest = e >> 2, row = rest >> lh, h2 = rest & (hpw - 1);
          const int fi = t0 + row;
          uint32_t off = kBwOob;
          if (fi < nrows) {
            const int m = fdiv(fi, a.f_n);
            off = (tok_off(a, mlist[m], fi - m * a.n) + (hg * hpw + h2) * kHd + 8 * c) * 2;
          }
          fq[u] = ld16(Qr, off);
          fg[u] = ld16(Gr, off);
        }
        float lv = 3.0e38f, dv = 0.f;                 // padding queries: p = 0
        if (tid < kDkvTile) {
          const int row = tid >> lh, h2 = tid & (hpw - 1), fi = t0 + row;
          if (fi < nrows) {
            const int m = fdiv(fi, a.f_n);
            const size_t pix = (size_t)b * a.H * a.W + tok_pix(a, mlist[m], fi - m * a.n);
            lv = a.lse[pix * a.heads + hg * hpw + h2];
            dv = a.dd[pix * a.heads + hg * hpw + h2];
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = tid + kThreads * u;
          const int c = e & 3, rest = e >> 2, row = rest >> lh, h2 = rest & (hpw - 1);
          *(uint4*)trow(tiles + h2 * TR * kHd, row, c) = fq[u];
          *(uint4*)trow(tiles + kDkvTile * kHd + h2 * TR * kHd, row, c) = fg[u];
        }
        if (tid < kDkvTile) {
          const int row = tid >> lh, h2 = tid & (hpw - 1);
          Ls0[h2 * TR + row] = lv;
          Ds0[h2 * TR + row] = dv;
        }
        __syncthreads();
        const int nsub = (min(TR, nrows - t0) + 31) / 32;
        if (act) {
          for (int hh = split; hh < nsub; hh += QS) {
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
        __syncthreads();                              // the tile is consumed
      }
    } while (e0 < RT);
    if (QS > 1) {
      // splits 1 .. QS-1 hand their sums to split 0 through the tile buffer
      // (free now): [QS - 1][roles][16][64] floats, at most 12 KB of its 16
      float* red = (float*)tiles;
      if (act && split > 0) {
        float* rw = red + ((split - 1) * roles + role) * 16 * 64 + lane;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rw[(e + 0) * 64] = ak0[e];
          rw[(e + 4) * 64] = ak1[e];
          rw[(e + 8) * 64] = av0[e];
          rw[(e + 12) * 64] = av1[e];
        }
      }
      __syncthreads();
      if (act && split == 0) {
        for (int sp = 1; sp < QS; ++sp) {
          const float* rr = red + ((sp - 1) * roles + role) * 16 * 64 + lane;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ak0[e] += rr[(e + 0) * 64];
            ak1[e] += rr[(e + 4) * 64];
            av0[e] += rr[(e + 8) * 64];
            av1[e] += rr[(e + 12) * 64];
          }
        }
      }
      __syncthreads();
    }
    if (kok && split == 0) {
      // lane holds channels 4 lg + e (acc 0) and 16 + 4 lg + e (acc 1) of key `key`
      const int to = tok_off(a, s, key) + h * kHd;
      float l0[4] = {0.f, 0.f, 0.f, 0.f}, l1[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.dv_lepe) {
        const float* lp = a.dv_lepe + (size_t)b * img + to + 4 * lg;
        const float4 x0 = *(const float4*)lp, x1 = *(const float4*)(lp + 16);
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

// The LePE gradients from one sliding window of dout.  Thread (channel pair
// cp, NCOL adjacent columns from x) of image b walks a strip of rows, holding
// the window G(i, j) = dout(y - i + P, x - j + P) (two bf16 channels a word;
// one such window per column); then
//   dV_L(y, x) = sum_{i,j} w(i, j) G(i, j)          (written as float32),
//   dw(i, j)  += V(y, x) G(i, j),   db += dout(y, x)
// (the second is the correlation sum over pixels with the centre moved to
// the V side).  Rows are fetched KS at a time, so that many loads are in
// flight per thread, and the window is a circular buffer of KS rows whose
// slot indices are compile-time in a KS-row batch: no data moves.  The
// workgroup's thread columns are added in LDS in column order and written as
// one row of part: [(b * nstrips + strip) * nxb + xb][C][KK + 1] (the KK
// taps, then db).  Consecutive threads take consecutive channel pairs of one
// pixel, so every load is coalesced.
// DwPlan, kMaxCols and dw_plan (the strip and column split) are host
// arithmetic in launch_plan.h.
static_assert(kThreads == kPlanThreads && kWaves == kPlanWaves, "launch_plan.h thread counts");

template <int KS, int NCOL>              // NCOL: adjacent pixel columns per thread
__global__ __launch_bounds__(kThreads) void lepe_bwd_kernel(const uint32_t* g, const uint32_t* v,
                                                            const float* w, int H, int W, int CP,
                                                            DwPlan pl, float* part, float* dvl) {
  constexpr int P = KS / 2, KK = KS * KS, NV = 2 * (KK + 1);
  __shared__ float red[32][kThreads];
  const int tid = threadIdx.x;
  const int cpl = tid % pl.cpb, xl = tid / pl.cpb;
  const int cp = blockIdx.y * pl.cpb + cpl;
  const int x = (blockIdx.x * pl.xc + xl) * NCOL;
  const int strip = blockIdx.z % pl.nstrips, b = blockIdx.z / pl.nstrips;
  const bool ok = xl < pl.xc && cp < CP && x < W;
  float acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = 0.f;
  if (ok) {
    const uint32_t iw = (uint32_t)H * W * CP;        // words of one image
    const auto Gr = rsrc(g + (size_t)b * iw, iw * 4), Vr = rsrc(v + (size_t)b * iw, iw * 4);
    float2* dl = (float2*)dvl + (size_t)b * iw + cp;
    // byte offset of word (y, x - P + c) of this channel pair, past the
    // record (reads zero) outside the image; unsigned arithmetic wraps back
    // to the right value for the columns that are inside
    constexpr int WC = KS + NCOL - 1;            // window columns
    const uint32_t rowb = (uint32_t)W * CP * 4, colb = (uint32_t)CP * 4;
    const uint32_t cb0 = ((uint32_t)(x - P) * CP + cp) * 4;
    bool colok[WC];
#pragma unroll
    for (int c = 0; c < WC; ++c) colok[c] = (unsigned)(x - P + c) < (unsigned)W;
    auto goff = [&](int y, int c) -> uint32_t {
      return ((unsigned)y < (unsigned)H && colok[c]) ? (uint32_t)y * rowb + cb0 + c * colb : kBwOob;
    };
    auto ldw = [&](__amdgpu_buffer_rsrc_t r, uint32_t o) -> uint32_t {
      return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
    };
    float w0[KK], w1[KK];                 // taps of channels 2 cp and 2 cp + 1
#pragma unroll
    for (int t = 0; t < KK; ++t) {
      w0[t] = w[(2 * cp) * KK + t];
      w1[t] = w[(2 * cp + 1) * KK + t];
    }
    const int y0 = strip * pl.sr, y1 = min(H, y0 + pl.sr);
    // circular window of dout rows: while row y = yb + u of a batch is
    // processed, row y - P + r sits in slot (u + r) % KS (r < KS), columns
    // x - P .. x + NCOL - 1 + P; a batch of KS rows returns the slots to
    // phase 0.  Up to 5 x 5 the window is held as floats (converted once per
    // load).
    constexpr bool FW = KS <= 5;
    float wf[FW ? KS : 1][FW ? WC : 1][2];
    uint32_t wu[FW ? 1 : KS][FW ? 1 : WC];
    auto put = [&](int r, int c, uint32_t u32) {
      if constexpr (FW) {
        wf[r][c][0] = bf16_lo(u32);
        wf[r][c][1] = bf16_hi(u32);
      } else {
        wu[r][c] = u32;
      }
    };
    auto get = [&](int r, int c, float& a0, float& a1) {
      if constexpr (FW) {
        a0 = wf[r][c][0];
        a1 = wf[r][c][1];
      } else {
        a0 = bf16_lo(wu[r][c]);
        a1 = bf16_hi(wu[r][c]);
      }
    };
#pragma unroll
    for (int r = 0; r + 1 < KS; ++r)
#pragma unroll
      for (int c = 0; c < WC; ++c) put(r, c, ldw(Gr, goff(y0 - P + r, c)));
    for (int yb = y0; yb < y1; yb += KS) {
      uint32_t nx[KS][WC], vc[KS][NCOL];         // the batch's new rows, in flight together
#pragma unroll
      for (int u = 0; u < KS; ++u) {
#pragma unroll
        for (int c = 0; c < WC; ++c) nx[u][c] = ldw(Gr, goff(yb + u + P, c));
#pragma unroll
        for (int o = 0; o < NCOL; ++o) vc[u][o] = ldw(Vr, goff(yb + u, P + o));
      }
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const int y = yb + u;
        const int sn = (KS - 1 + u) % KS;             // slot of the new row y + P
#pragma unroll
        for (int c = 0; c < WC; ++c) put(sn, c, nx[u][c]);
        // rows past the strip (and columns past the image) are computed with
        // zero weight and not stored
        const float fv = y < y1 ? 1.f : 0.f;
#pragma unroll
        for (int o = 0; o < NCOL; ++o) {
          const float v0 = bf16_lo(vc[u][o]) * fv, v1 = bf16_hi(vc[u][o]) * fv;
          float l0 = 0.f, l1 = 0.f;
#pragma unroll
          for (int i = 0; i < KS; ++i) {
            const int sl = (u + KS - 1 - i) % KS;     // dout row y - i + P
#pragma unroll
            for (int j = 0; j < KS; ++j) {
              float g0, g1;
              get(sl, KS - 1 - j + o, g0, g1);        // dout(y - i + P, x + o - j + P)
              const int t = i * KS + j;
              l0 = fmaf(w0[t], g0, l0);
              l1 = fmaf(w1[t], g1, l1);
              acc[2 * t] = fmaf(v0, g0, acc[2 * t]);
              acc[2 * t + 1] = fmaf(v1, g1, acc[2 * t + 1]);
            }
          }
          const float fo = colok[P + o] ? fv : 0.f;
          float gc0, gc1;
          get((u + P) % KS, P + o, gc0, gc1);         // dout(y, x + o)
          acc[2 * KK] = fmaf(fo, gc0, acc[2 * KK]);
          acc[2 * KK + 1] = fmaf(fo, gc1, acc[2 * KK + 1]);
          if (y < y1 && colok[P + o]) dl[(size_t)(y * W + x + o) * CP] = make_float2(l0, l1);
        }
      }
    }
  }
  // column sums: item (j, pair) of a 32-value slice, one per thread at a
  // time, the xc columns (at most kMaxCols) added in column order
  float* pr = part + ((size_t)blockIdx.z * gridDim.x + blockIdx.x) * (size_t)(2 * CP) * (KK + 1);
#pragma unroll
  for (int c0 = 0; c0 < NV; c0 += 32) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (c0 + j < NV) red[j][tid] = acc[c0 + j];
    __syncthreads();
    for (int it = tid; it < 32 * pl.cpb; it += kThreads) {
      const int j = it / pl.cpb, pc = it - j * pl.cpb, cpp = blockIdx.y * pl.cpb + pc;
      if (c0 + j < NV && cpp < CP) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxCols; ++q)
          if (q < pl.xc) sum += red[j][q * pl.cpb + pc];
        const int vi = c0 + j, t = vi >> 1, half = vi & 1;
        pr[(2 * cpp + half) * (KK + 1) + t] = sum;
      }
    }
    __syncthreads();
  }
}

// dw[c][t] and db[c]: float64 sums of the partial rows.  A workgroup takes 8
// columns of part with 32 row phases each; the phases are added in order.
__global__ __launch_bounds__(kThreads) void lepe_dw_sum_kernel(const float* part, long long rows,
                                                               int CT, int KK, float* dw,
                                                               float* db) {
  __shared__ double red[32][8];
  const int cl = threadIdx.x & 7, ph = threadIdx.x >> 3;
  const int col = blockIdx.x * 8 + cl;
  double s = 0.0;
  if (col < CT) {
    long long r = ph;
    for (; r + 7 * 32 < rows; r += 8 * 32) {       // eight loads in flight, added in order
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = part[(size_t)(r + 32 * u) * CT + col];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += t[u];
    }
    for (; r < rows; r += 32) s += part[(size_t)r * CT + col];
  }
  red[ph][cl] = s;
  __syncthreads();
  if (ph == 0 && col < CT) {
    double t = 0.0;
    for (int p = 0; p < 32; ++p) t += red[p][cl];
    const int c = col / (KK + 1), tt = col - c * (KK + 1);
    if (tt < KK) dw[c * KK + tt] = (float)t;
    else if (db) db[c] = (float)t;
  }
}

}  // namespace

hipError_t launch_backward(const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* dout, const Shape& s, float attn_scale, const float* w,
                           int ks, void* dq, void* dk, void* dvv, float* dw, float* db, void* ws,
                           hipStream_t st) {
  if (s.C != s.heads * kHd || s.topk * s.n > kBwMaxKeys) return hipErrorNotSupported;
  if (w && (ks < 1 || ks > 7 || ks % 2 == 0)) return hipErrorInvalidValue;
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
  a.f_S = make_fastdiv(s.S);
  a.f_ws = make_fastdiv(s.ws);
  a.f_n = make_fastdiv(s.n);
  a.f_topk = make_fastdiv(s.topk);
  a.f_R = make_fastdiv(s.R);
  const size_t px = (size_t)s.B * s.H * s.W;
  unsigned char* w8 = (unsigned char*)ws;
  a.lse = (float*)w8;
  a.dd = a.lse + px * s.heads;
  size_t used = 2 * px * s.heads * sizeof(float);
  used = (used + 255) / 256 * 256;
  hipError_t e;
  const unsigned units = (unsigned)(s.B * s.R * s.heads);
  a.dv_lepe = nullptr;
  // LePE: dV's LePE term (float32, added by bwd_dkv_kernel), dw, db
  if (w) {
    const DwPlan pl = dw_plan(s.B, s.H, s.W, s.C, ks);
    if ((long long)s.B * pl.nstrips > 65535 || pl.ncb > 65535) return hipErrorNotSupported;
    float* dvl = (float*)(w8 + used);
    float* part = dvl + px * s.C;
    a.dv_lepe = dvl;
    const dim3 g1((unsigned)pl.nxb, (unsigned)pl.ncb, (unsigned)(s.B * pl.nstrips));
    const uint32_t* g32 = (const uint32_t*)dout;
    const uint32_t* v32 = (const uint32_t*)v;
#define BRA_LEPE_BW(KSV) \
    hipLaunchKernelGGL((lepe_bwd_kernel<KSV, KSV <= 5 ? 2 : 1>), g1, dim3(kThreads), 0, st, g32, \
                       v32, w, s.H, s.W, s.C / 2, pl, part, dvl)
    switch (ks) {
      case 1: BRA_LEPE_BW(1); break;
      case 3: BRA_LEPE_BW(3); break;
      case 5: BRA_LEPE_BW(5); break;
      default: BRA_LEPE_BW(7); break;
    }
#undef BRA_LEPE_BW
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int KK = ks * ks, CT = s.C * (KK + 1);
    hipLaunchKernelGGL(lepe_dw_sum_kernel, dim3((unsigned)((CT + 7) / 8)), dim3(kThreads), 0, st,
                       part, pl.rows, CT, KK, dw, db);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dq (and the saved statistics), then dk / dv
  // heads per workgroup: small regions leave wavefronts without a query
  // block (dq) or key block (dk, dv) of their own; they take more heads
  const int NH = (s.topk * s.n + 31) / 32;
  const int nqb = (s.n + 15) / 16, KB = nqb;
  int hq = 1, hk = 1;
  for (int c = kWaves; c > 1; c /= 2) {
    if (hq == 1 && nqb * c <= kWaves && s.heads % c == 0 && 32 * NH * c <= 512) hq = c;
    if (hk == 1 && KB * c <= kWaves && s.heads % c == 0) hk = c;
  }
  const size_t lq = (size_t)2 * hq * 32 * NH * kHd * 2;
  const bool full = (s.topk * s.n) % 32 == 0;
  const void* dqf = full ? (const void*)bwd_dq_kernel<true> : (const void*)bwd_dq_kernel<false>;
  e = hipFuncSetAttribute(dqf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lq);
  if (e != hipSuccess) return e;
  if (full)
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3(units / hq), dim3(kThreads), lq, st, a, NH, hq);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3(units / hq), dim3(kThreads), lq, st, a, NH, hq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3(units / hk), dim3(kThreads), 0, st, a, hk);
  return hipGetLastError();
}

}  // namespace bra
