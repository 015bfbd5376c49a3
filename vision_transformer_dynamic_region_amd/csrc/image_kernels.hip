// Gather-attention + LePE with the whole image's keys and values resident in
// LDS, for bf16 maps small enough that one head of one image fits there (the
// BiFormer stage-2 and stage-3 shapes at a 224^2 input: 28x28 and 14x14 maps
// cut into 7x7 regions of 4x4 and 2x2 pixels, routed to 4 and 16 regions).
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3: the routed regions' tokens are gathered, softmax attention runs over
// them, LePE is added to the output), p2 = snabindia.com "从静态到动态：BRA双
// 层路由注意力如何革新视觉Transformer的计算范式" (§4: torch.gather copies the
// routed keys top-k times over; the LePE depthwise conv on V), p5 = hyper.ai
// abstract of BiFormer (token-to-token attention over the union of the routed
// regions).
//
// With small regions and a large top-k every key region is routed to by many
// query regions (16 on average at stage 3), so a per-region gather moves
// each key top-k times through L2.  Here a workgroup owns one head of one
// image (or a range of its query regions): it stages that head's K (in
// region-major order) and V (as the image with a zero border of KS/2 pixels,
// which is also the LePE halo of every region) into LDS once, and then the
// gather is LDS addressing: each lane computes the address of its own routed
// key rows from the routing table.  Per task (one query region, 16 query
// columns, this head), on one wavefront and with no barrier:
//   attention  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows read at the
//              routed positions), softmax numerators in float32 with the
//              scale folded into exp2, rounded to bf16; O^T = V^T P^T with the
//              V^T operands read by transposing LDS reads at the routed
//              pixels; row sums by an MFMA against a ones operand;
//   LePE       5x5 cross-correlation of the padded V image on
//              v_dot2_f32_bf16 (tap pairs along x, weights rounded once to
//              bf16, products exact, float32 sums), interleaved with the
//              attention phases;
//   epilogue   L through a wavefront-private LDS tile into the MFMA layout,
//              out = O / l + L rounded once to bf16, 16-byte stores.
// Q is read straight into registers, one task ahead.

#include "device_common.h"

namespace bra {
namespace {

constexpr int kHd = 32;   // head width = channels a workgroup owns

template <int HS_, int WS_, int TOPK_, int KS_, int NW_>
struct Ic {
  // HS x WS pixels a region, TOPK routed regions, KS x KS LePE, NW
  // wavefronts a workgroup
  static constexpr int HS = HS_, WS = WS_, TOPK = TOPK_, KS = KS_, NW = NW_;
  static constexpr int NT = NW * 64;                   // threads
  static constexpr int n = HS * WS;                    // queries (and keys) per region
  static constexpr int KC = TOPK * n;                  // routed keys of a query region
  static constexpr int NQB = (n + 15) / 16;            // 16-query blocks per region
  static constexpr int P = KS / 2, KK = KS * KS;
  // LePE items of a wavefront: 32 channels x 16 query pixels, two items per
  // channel lane, each XG columns (tap pairs along x) by TYW rows
  static constexpr int QR = (n < 16 ? n : 16) / WS;    // pixel rows of a query block
  static constexpr int XG = WS % 4 == 0 ? 4 : WS;
  static constexpr int NXG = WS / XG;
  static constexpr int TYW = QR * NXG / 2;
  static constexpr int LSW = kHd + 4;                  // L tile row stride (floats)
  static constexpr int NB = 4;                         // staging vectors in flight a thread (K and V each)
  static_assert(KC % 32 == 0 && KC <= 256, "routed keys: a multiple of 32, one softmax step");
  static_assert(n >= 16 ? 16 % WS == 0 : n % WS == 0, "query blocks are whole pixel rows");
  static_assert(KS == 5 && (XG == 4 || XG == 2) && TYW >= 1 && (QR * NXG) % 2 == 0,
                "LePE: 5x5 taps read as 8-pixel rows, two items per channel lane");
};

struct ImageArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  const float* w;       // [C, KS, KS]
  const float* bias;    // [C] or null
  int B, H, W, C, S, R, heads;
  int rsplit;           // workgroups per (image, head), each a range of query regions
  int rper;             // query regions per workgroup
  float scale_log2;     // attn_scale * log2(e)
  int ks_off, vs_off, it_off, lw_off, wt_off;   // LDS byte offsets
  FastDiv f_S, f_W, f_rsplit, f_heads, f_wp4;   // f_wp4: (W + 2P) * 4 (padded pixel chunks)
};

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr uint32_t kOob = 0x80000000u;           // byte offset outside every image
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t image_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, BRA_OUT_CPOL);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// K tile: key position pos (region-major), 16-byte chunk g at g ^ kswz(pos):
// eight consecutive positions reading one chunk hit eight distinct 16-byte
// bank groups (two positions share a 128-byte bank row).
__device__ __forceinline__ int kswz(int pos) { return (pos >> 1) & 3; }
// V image (padded pixel py, px): the two 32-byte halves of a pixel swap when
// bit 0 of py ^ (px >> 1) is set, so four consecutive pixels of a row, or
// the 2x2 pixels of a region, read by one transposing read hit four distinct
// 32-byte bank groups.
__device__ __forceinline__ int vswz(int py, int px) { return ((py ^ (px >> 1)) & 1) << 1; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <class G>
__global__ __launch_bounds__(G::NT) void attend_image_kernel(ImageArgs A) {
  constexpr int HS = G::HS, WS = G::WS, TOPK = G::TOPK, KS = G::KS, NW = G::NW, NT = G::NT;
  constexpr int n = G::n, KC = G::KC, NQB = G::NQB, P = G::P, KK = G::KK;
  constexpr int XG = G::XG, NXG = G::NXG, TYW = G::TYW, LSW = G::LSW, NB = G::NB;
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Ks = (uint16_t*)(lds + A.ks_off);
  uint16_t* Vs = (uint16_t*)(lds + A.vs_off);
  int2* itab = (int2*)(lds + A.it_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // tasks are wavefront-uniform
  const int lq = lane & 15, lg = lane >> 4;
  // workgroup -> (image, head, region range); every workgroup of an image
  // sits on the image's XCD (blockIdx % 8), so its L2 serves whole lines
  const int xcd = blockIdx.x % kXcds, rest = blockIdx.x / kXcds;
  const int t1 = fdiv(rest, A.f_rsplit), rs = rest - t1 * A.rsplit;
  const int t2 = fdiv(t1, A.f_heads), h = t1 - t2 * A.heads;
  const int b = t2 * kXcds + xcd;
  if (b >= A.B) return;                              // uniform over the workgroup
  const int r0 = rs * A.rper;
  const int r1 = min(A.R, r0 + A.rper);
  if (r0 >= r1) return;

  const int H = A.H, W = A.W, C = A.C, S = A.S;
  const int WP = W + 2 * P, HP = H + 2 * P;
  const uint32_t img_elems = (uint32_t)H * W * C;
  const size_t img = (size_t)b * img_elems;
  const auto Qr = image_rsrc(A.q + img, img_elems * 2);
  const auto Kr = image_rsrc(A.k + img, img_elems * 2);
  const auto Vr = image_rsrc(A.v + img, img_elems * 2);
  const auto Or = image_rsrc(A.out + img, img_elems * 2);
  const int c0 = h * kHd;

  const int cw = lane & 31;
  const int ntask = (r1 - r0) * NQB;
  auto q_off = [&](int task) -> uint32_t {
    const int rl = task / NQB, qb = task - rl * NQB;
    const int r = r0 + rl;
    const int ry = fdiv(r, A.f_S), rx = r - ry * S;
    const int q = qb * 16 + lq;
    const uint32_t off = ((ry * HS + q / WS) * W + rx * WS + q % WS) * C + c0 + 8 * lg;
    return q < n ? off * 2 : kOob;
  };
  int task = wave;
  uint4 qn;

  // ---- stage: K region-major, V into the padded image, routing rows.  The
  // routing entries, this lane's LePE weights and the first task's Q are
  // issued while the first round of K and V chunks is in flight, and the
  // zero border of the V image is written meanwhile, so the staging waits
  // on one round trip to memory, not three ----
  const int nent = (r1 - r0) * TOPK;
  const int32_t* irow = A.idx + ((size_t)b * A.R + r0) * TOPK;
  int ent0 = 0;
  // this head's LePE weights ([32 channels][KK] floats, one contiguous run
  // of memory) are read in order by the workgroup and kept in LDS
  constexpr int NWT = (KK * kHd + NT - 1) / NT;
  float wv[NWT];
  float* wtab = (float*)(lds + A.wt_off);
  {
    const int total = H * W * 4;                     // 16-byte chunks of this head
    for (int e0 = 0; e0 < total; e0 += NB * NT) {
      uint4 kr[NB], vr[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = e0 + i * NT + tid;
        const int p = e >> 2, g = e & 3;
        const uint32_t off = e < total ? (uint32_t)(p * C + c0 + g * 8) * 2 : kOob;
        kr[i] = bload16(Kr, off);
        vr[i] = bload16(Vr, off);
      }
      if (e0 == 0) {
        ent0 = tid < nent ? irow[tid] : 0;
        const float* wsrc = A.w + (size_t)c0 * KK;
#pragma unroll
        for (int i = 0; i < NWT; ++i) {
          const int e = i * NT + tid;
          wv[i] = e < KK * kHd ? wsrc[e] : 0.f;
        }
        qn = bload16(Qr, task < ntask ? q_off(task) : kOob);
        // the zero border of the V image (position within a pixel does not matter)
        for (int e = tid; e < HP * WP * 4; e += NT) {
          const int pc = fdiv(e, A.f_wp4);             // padded row
          const int px = (e - pc * WP * 4) >> 2;
          if ((unsigned)(pc - P) >= (unsigned)H || (unsigned)(px - P) >= (unsigned)W)
            *(uint4*)(Vs + e * 8) = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int e = e0 + i * NT + tid;
        if (e < total) {
          const int p = e >> 2, g = e & 3;
          const int y = fdiv(p, A.f_W), x = p - y * W;
          const int ry = y / HS, ty = y - ry * HS, rx = x / WS, tx = x - rx * WS;
          const int pos = (ry * S + rx) * n + ty * WS + tx;
          *(uint4*)(Ks + pos * kHd + ((g ^ kswz(pos)) << 3)) = kr[i];
          const int py = y + P, px = x + P;
          *(uint4*)(Vs + (py * WP + px) * kHd + ((g ^ vswz(py, px)) << 3)) = vr[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NWT; ++i) {
      const int e = i * NT + tid;
      if (e < KK * kHd) wtab[e] = wv[i];
    }
    // routing rows of this workgroup's query regions: the routed region's
    // first key position and the padded image coordinates of its top-left
    // pixel (indices clamped into [0, R)); entry tid came with the staging
    for (int e = tid; e < nent; e += NT) {
      const int reg = min(max(e == tid ? ent0 : irow[e], 0), A.R - 1);
      const int sy = fdiv(reg, A.f_S), sx = reg - sy * S;
      itab[e] = make_int2(reg * n, ((sy * HS + P) << 16) | (sx * WS + P));
    }
  }

  const float b0 = A.bias ? A.bias[c0 + cw] : 0.f;
  __syncthreads();
  // this channel lane's LePE weights as bf16 pairs per kernel row i: for an
  // even output column the tap pairs (w0,w1) (w2,w3) (w4,0) over pixel pairs
  // (x,x+1) (x+2,x+3) (x+4,x+5); for the odd column after it (0,w0) (w1,w2)
  // (w3,w4) over the same pairs
  uint32_t we[KS][3], wo[KS][3];
  {
    const float* wt = wtab + cw * KK;               // KK odd: lanes hit distinct banks
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const float t0 = wt[i * KS], t1 = wt[i * KS + 1], t2 = wt[i * KS + 2];
      const float t3 = wt[i * KS + 3], t4 = wt[i * KS + 4];
      we[i][0] = pack_bf16x2(t0, t1);
      we[i][1] = pack_bf16x2(t2, t3);
      we[i][2] = pack_bf16x2(t4, 0.f);
      wo[i][0] = pack_bf16x2(0.f, t0);
      wo[i][1] = pack_bf16x2(t1, t2);
      wo[i][2] = pack_bf16x2(t3, t4);
    }
  }

  const float c = A.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u, 0x3f803f80u));
  float* Lw = (float*)(lds + A.lw_off) + wave * 16 * LSW;   // this wavefront's L tile
  const int grp = lane >> 5;
  const int xw = (grp % NXG) * XG, yl = (grp / NXG) * TYW;

  for (; task < ntask; task += NW) {
    const bf16x8 qop = __builtin_bit_cast(bf16x8, qn);
    // the next task's Q, always issued (past the range it reads zeros)
    qn = bload16(Qr, task + NW < ntask ? q_off(task + NW) : kOob);
    const int rl = task / NQB, qb = task - rl * NQB;
    const int r = r0 + rl;
    const int ry = fdiv(r, A.f_S), rx = r - ry * S;
    const int qrow0 = qb * 16 / WS;
    const int2* it = itab + rl * TOPK;

    // ---- LePE of this lane's items, in three slices of input rows ----
    float lw[TYW][XG];
#pragma unroll
    for (int rr = 0; rr < TYW; ++rr)
#pragma unroll
      for (int kx = 0; kx < XG; ++kx) lw[rr][kx] = b0;
    // transposing reads of 4 consecutive padded pixels of one channel: lane
    // i of a 16-lane row addresses pixel x + i/4 (+4 for the second read),
    // channels (cw & ~15) + 4(i % 4) .. +3, and receives channel cw of the
    // four pixels as two bf16 pairs along x; the taps are dot2 products of
    // those pairs with the weight pairs
    const int cq = (cw & ~15) + 4 * (lane & 3);       // first channel addressed
    const int py0 = ry * HS + qrow0 + yl;             // padded row of tap row 0
    const int pxa = rx * WS + xw + (lq >> 2), pxb = pxa + 4;
    auto conv_rows = [&](int dy0, int dy1) {
#pragma unroll
      for (int dy = 0; dy < TYW + KS - 1; ++dy) {
        if (dy < dy0 || dy >= dy1) continue;
        const int py = py0 + dy;
        const uint2 a = lds_read_tr16(Vs + (py * WP + pxa) * kHd +
                                      (((cq >> 3) ^ vswz(py, pxa)) << 3) + (cq & 7));
        const uint2 bb = lds_read_tr16(Vs + (py * WP + pxb) * kHd +
                                       (((cq >> 3) ^ vswz(py, pxb)) << 3) + (cq & 7));
        // pixel pairs (x,x+1) .. (x+6,x+7) of this tap row (the last unused
        // when XG == 2)
        const uint32_t p0 = a.x, p1 = a.y, p2 = bb.x, p3 = bb.y;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const int rr = dy - i;
          if (rr < 0 || rr >= TYW) continue;
          lw[rr][0] = dot2(we[i][2], p2, dot2(we[i][1], p1, dot2(we[i][0], p0, lw[rr][0])));
          lw[rr][1] = dot2(wo[i][2], p2, dot2(wo[i][1], p1, dot2(wo[i][0], p0, lw[rr][1])));
          if constexpr (XG == 4) {
            lw[rr][2] = dot2(we[i][2], p3, dot2(we[i][1], p2, dot2(we[i][0], p1, lw[rr][2])));
            lw[rr][3] = dot2(wo[i][2], p3, dot2(wo[i][1], p2, dot2(wo[i][0], p1, lw[rr][3])));
          }
        }
      }
    };
    constexpr int NR = TYW + KS - 1;                  // input rows of an item

    // ---- attention phase 1: S^T = K Q^T over the routed key positions ----
    float x[KC / 4];
#pragma unroll
    for (int kb = 0; kb < KC / 16; ++kb) {
      const int key = 16 * kb + lq;
      const int pos = it[key / n].x + key % n;
      const bf16x8 ka = *(const bf16x8*)(Ks + pos * kHd + ((lg ^ kswz(pos)) << 3));
      const f32x4 sv = mfma_bf16(ka, qop, f32x4{0.f, 0.f, 0.f, 0.f});
      // lane holds keys 16*kb + 4*lg + e of query lq
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * kb + e] = sv[e];
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(0, NR / 3);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2: softmax numerators, rounded to bf16 in P^T slot order ----
    uint32_t ph[KC / 8];
    {
      float m = x[0];
#pragma unroll
      for (int e = 1; e < KC / 4; ++e) m = fmaxf(m, x[e]);
      m = fmaxf(m, xor16(m));
      m = fmaxf(m, xor32(m));
      const float mc = m * c;
#pragma unroll
      for (int e = 0; e < KC / 8; ++e)
        ph[e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(x[2 * e], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(x[2 * e + 1], c, -mc)));
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(NR / 3, 2 * NR / 3);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 3: O^T += V^T P^T, row sums += ones P^T ----
    // lane (lq, lg) addresses routed key 32h + 4lg + lq/4 (+16 for slots
    // 4-7), channels d0 + 4(lq % 4) .. +3 of its padded pixel, and receives
    // channel d0 + lq of keys 4lg + 0..3: the slot order of P^T
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
    {
      const int cc = 4 * (lq & 3);                    // channel within a 16-channel half
#pragma unroll
      for (int hh = 0; hh < KC / 32; ++hh) {
        const uint16_t* vrow[2];
        int vsw[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int key = 32 * hh + 16 * s2 + 4 * lg + (lq >> 2);
          const int t = key % n;
          const int pc = it[key / n].y;
          const int py = (pc >> 16) + t / WS, px = (pc & 0xffff) + t % WS;
          vrow[s2] = Vs + (py * WP + px) * kHd;
          vsw[s2] = vswz(py, px);
        }
        const int ga = cc >> 3, gb = (16 + cc) >> 3, wi = cc & 7;
        const uint2 a0 = lds_read_tr16(vrow[0] + ((ga ^ vsw[0]) << 3) + wi);
        const uint2 a1 = lds_read_tr16(vrow[1] + ((ga ^ vsw[1]) << 3) + wi);
        const uint2 d0 = lds_read_tr16(vrow[0] + ((gb ^ vsw[0]) << 3) + wi);
        const uint2 d1 = lds_read_tr16(vrow[1] + ((gb ^ vsw[1]) << 3) + wi);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
        const bf16x8 phi = __builtin_bit_cast(
            bf16x8, make_uint4(ph[4 * hh], ph[4 * hh + 1], ph[4 * hh + 2], ph[4 * hh + 3]));
        acc0 = mfma_bf16(va, phi, acc0);               // O^T rows d = 4lg + e
        acc1 = mfma_bf16(vb, phi, acc1);               // O^T rows d = 16 + 4lg + e
        accl = mfma_bf16(ones, phi, accl);             // every row: sum over keys
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(2 * NR / 3, NR);

    // ---- L through the wavefront's tile into the MFMA layout ----
#pragma unroll
    for (int rr = 0; rr < TYW; ++rr)
#pragma unroll
      for (int kx = 0; kx < XG; ++kx) Lw[((yl + rr) * WS + xw + kx) * LSW + cw] = lw[rr][kx];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- out = O / l + L, one rounding, 16-byte stores ----
    {
      const int q = qb * 16 + lq;
      const float inv = __builtin_amdgcn_rcpf(accl[0]);
      const float* lp = Lw + (q < n ? lq : 0) * LSW;     // pixels past n: not stored
      const float4 a0 = *(const float4*)(lp + 4 * lg);
      const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
      const uint32_t o0x = pack_bf16x2(fmaf(acc0[0], inv, a0.x), fmaf(acc0[1], inv, a0.y));
      const uint32_t o0y = pack_bf16x2(fmaf(acc0[2], inv, a0.z), fmaf(acc0[3], inv, a0.w));
      const uint32_t o1x = pack_bf16x2(fmaf(acc1[0], inv, a1.x), fmaf(acc1[1], inv, a1.y));
      const uint32_t o1y = pack_bf16x2(fmaf(acc1[2], inv, a1.z), fmaf(acc1[3], inv, a1.w));
      // lane rows lg, lg^1 trade halves: even rows end up with channels
      // 4lg..4lg+7, odd rows with 16+4(lg-1)..16+4lg+3 -- 16 contiguous bytes
      const auto sx = __builtin_amdgcn_permlane16_swap(o0x, o1x, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(o0y, o1y, false, false);
      const bool odd = lg & 1;
      const uint4 ov = odd ? make_uint4(sx[0], sy[0], o1x, o1y) : make_uint4(o0x, o0y, sx[1], sy[1]);
      const int ch = odd ? 16 + 4 * (lg - 1) : 4 * lg;
      const uint32_t op = ((ry * HS + q / WS) * W + rx * WS + q % WS) * C + c0 + ch;
      bstore16(Or, q < n ? op * 2 : kOob, ov);
    }
    // the L tile is rewritten by this wavefront's next task only after its
    // reads above (program order within the wavefront)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// 2x2-pixel regions.  A 16-query MFMA column block holds four whole query
// regions, and the block is evaluated against every key of the image with
// the routing applied as a per-(query region, key region) multiplicity
// (0 for regions not routed to; a region listed twice counts twice, as its
// keys would in a gather).  With four queries a region the per-region form
// pads each 16-column block to four times its queries, so for 49 regions
// routed to 16 this costs fewer matrix operations and softmax values than
// the gather (208 x 224 logits an image and head against 49 x 16 x 64) and
// reads K and V rows in order.  Per block, on one wavefront:
//   pass 1     S^T = K Q^T over the key blocks, the maximum of the routed
//              logits;
//   pass 2     S^T again, p = count * 2^(s c - m c) rounded to bf16, and per
//              32 keys O^T += V^T P^T and the row sums += ones P^T;
//   LePE       the block's 16 pixels from the padded V image: tap pairs along
//              x on v_dot2_f32_bf16 (weights rounded to bf16, products exact,
//              float32 sums);
//   epilogue   out = O / l + L, one rounding, 16-byte stores.
//
// Grouped form (GROUP): the same staging and LePE, but each query column
// meets only the keys its own region is routed to.  The four query regions
// of a block each bring their routed key rows (read at the routed positions
// in LDS); S^T for 16 routed keys is the sum of four MFMAs whose Q operand
// keeps only the columns of one region (the other columns are zero), so
// every column ends with the logits of its own region's keys, and O^T and
// the row sums are built the same way from V^T rows gathered per region and
// P^T operands keeping one region's columns.  A query then takes 4 TOPK
// softmax values instead of one per key of the image (st3: 64 against 224),
// at four MFMAs per 16 keys; the exponentials are what the masked form is
// bound by.
// ---------------------------------------------------------------------------
template <int TOPK_, int NW_, int NKB2_, bool GROUP_ = false>
struct Im {
  // TOPK routed regions, NW wavefronts a workgroup, NKB2 steps of 32 keys
  // (the image's keys padded to a multiple of 32)
  static constexpr int HS = 2, WS = 2, n = 4, TOPK = TOPK_, KS = 5, NW = NW_, NKB2 = NKB2_;
  static constexpr bool GROUP = GROUP_;
  static constexpr int KB = TOPK / 4;                 // (GROUP) 16-key blocks of a region's keys
  // (GROUP) byte offset of the V rows: right after the K rows at offset 0;
  // they are kept as two arrays of 16-channel halves [pos][16], VH bytes
  // each, so a transposing read of either half is one address apart
  static constexpr int VS_OFF = 32 * NKB2 * kHd * 2;
  static constexpr int VH = 32 * NKB2 * 16 * 2;
  static constexpr int NKB = 2 * NKB2;                // 16-key blocks
  static constexpr int NT = NW * 64, P = KS / 2, KK = KS * KS, LSW = kHd + 4;
  static constexpr int NBS = (128 * NKB2 + NT - 1) / NT;   // K (and V) chunks a thread stages
  static constexpr int NES = (64 * TOPK + NT - 1) / NT;    // routing entries a thread (R <= 64)
  static_assert(KS == 5 && NT >= KS * 3 * kHd, "LePE weights: one tap-pair entry a thread");
  static_assert(!GROUP || (TOPK % 8 == 0 && TOPK * 4 <= 64),
                "grouped form: whole 32-key steps, a routing row within a table row");
};

struct MaskArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  const float* w;       // [C, KS, KS]
  const float* bias;    // [C] or null
  int B, H, W, C, S, R, heads;
  int nqb;              // 16-query blocks per image (4 regions each)
  int nkb;              // 16-key blocks per image (keys padded to 32 in LDS; unused)
  int qsplit;           // workgroups per (image, head), each a range of query blocks
  int qper;             // query blocks per workgroup
  float scale_log2;     // attn_scale * log2(e)
  int ks_off, vs_off, vi_off, ct_off, rt_off, ws_off, lw_off;   // LDS byte offsets
  FastDiv f_S, f_W, f_qsplit, f_heads, f_wp4;
};

// V rows in region-major order: the two 32-byte halves of a row swap when
// bit 1 of its position is set, so the four rows one transposing read
// addresses (two consecutive pairs) hit four distinct 32-byte bank groups.
__device__ __forceinline__ int vrswz(int pos) { return ((pos >> 1) & 1) << 1; }
// Padded V image of the masked form: the halves of a pixel swap when bit 1
// of its column is set, so the four consecutive pixels of one row that 16
// lanes read for a LePE tap row hit four distinct 32-byte bank groups (rows
// do not share a read, so the row takes no part).
__device__ __forceinline__ int vmswz(int px) { return ((px >> 1) & 1) << 1; }


template <class G>
__global__ __launch_bounds__(G::NT) void attend_image_mask_kernel(MaskArgs A) {
  constexpr int TOPK = G::TOPK, KS = G::KS, NW = G::NW, NT = G::NT, n = G::n;
  constexpr int P = G::P, KK = G::KK, LSW = G::LSW, NKB = G::NKB, NKB2 = G::NKB2;
  constexpr int NBS = G::NBS, NES = G::NES;
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* Ks = (uint16_t*)(lds + A.ks_off);       // [32 NKB2][32] region-major
  uint16_t* Vs = (uint16_t*)(lds + A.vs_off);       // the same rows of V
  uint16_t* Vi = (uint16_t*)(lds + A.vi_off);       // the padded V image
  unsigned char* ct = lds + A.ct_off;               // [query region][4][16] multiplicities
  int* rtab = (int*)(lds + A.rt_off);               // per region: LePE base address
  uint2* wpr = (uint2*)(lds + A.ws_off);            // LePE dot2 weights [KS][3][32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 15, lg = lane >> 4;
  const int xcd = blockIdx.x % kXcds, rest = blockIdx.x / kXcds;
  const int t1 = fdiv(rest, A.f_qsplit), qs = rest - t1 * A.qsplit;
  const int t2 = fdiv(t1, A.f_heads), h = t1 - t2 * A.heads;
  const int b = t2 * kXcds + xcd;
  if (b >= A.B) return;                              // uniform over the workgroup
  const int qb0 = qs * A.qper;
  const int qb1 = min(A.nqb, qb0 + A.qper);
  if (qb0 >= qb1) return;
  const int qr0 = 4 * qb0;                           // first query region of the range
  const int nqr = min(A.R, 4 * qb1) - qr0;           // query regions of the range

  const int H = A.H, W = A.W, C = A.C, S = A.S, R = A.R;
  const int WP = W + 2 * P, HP = H + 2 * P;
  const int nkeys = R * n;
  const uint32_t img_elems = (uint32_t)H * W * C;
  const size_t img = (size_t)b * img_elems;
  const auto Qr = image_rsrc(A.q + img, img_elems * 2);
  const auto Kr = image_rsrc(A.k + img, img_elems * 2);
  const auto Vr = image_rsrc(A.v + img, img_elems * 2);
  const auto Or = image_rsrc(A.out + img, img_elems * 2);
  const int c0 = h * kHd;

  // this lane's query: region 4 qb + lq / 4, token lq % 4
  auto q_off = [&](int qb) -> uint32_t {
    const int qr = 4 * qb + (lq >> 2), t = lq & 3;
    const int ry = fdiv(min(qr, R - 1), A.f_S), rx = min(qr, R - 1) - ry * S;
    const uint32_t off = ((ry * 2 + (t >> 1)) * W + rx * 2 + (t & 1)) * C + c0 + 8 * lg;
    return qr < R ? off * 2 : kOob;
  };
  int qb = qb0 + wave;
  uint4 qn = bload16(Qr, qb < qb1 ? q_off(qb) : kOob);

  // ---- stage.  Every global read is issued first (K and V rows, the LePE
  // weights, the routing entries), the LDS areas that are only cleared are
  // cleared while they are in flight, then the loaded values are written ----
  const int cw = lane & 31;
  {
    const int total = H * W * 4;                     // 16-byte chunks of this head (<= 128 NKB2)
    uint4 kr[NBS], vr[NBS];
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      const int e = i * NT + tid;
      const uint32_t off = e < total ? (uint32_t)((e >> 2) * C + c0 + (e & 3) * 8) * 2 : kOob;
      kr[i] = bload16(Kr, off);
      vr[i] = bload16(Vr, off);
    }
    // one (kernel row, tap pair) entry of this head's LePE weights a thread
    const int we = tid;
    float wt[KS] = {};
    if (we < KS * 3 * kHd) {
      const float* wr = A.w + (size_t)(c0 + (we & 31)) * KK + ((we >> 5) / 3) * KS;
#pragma unroll
      for (int jx = 0; jx < KS; ++jx) wt[jx] = wr[jx];
    }
    // routing entries of the range's query regions, one a thread and step
    const int nent = nqr * TOPK;
    const auto Ir = image_rsrc(A.idx + ((size_t)b * R + qr0) * TOPK, (uint32_t)nent * 4);
    int ent[NES];
#pragma unroll
    for (int i = 0; i < NES; ++i) {
      const int e = i * NT + tid;
      ent[i] = __builtin_amdgcn_raw_buffer_load_b32(Ir, e < nent ? (uint32_t)e * 4 : kOob, 0, 0);
    }
    // cleared areas: key rows past the last key (their multiplicity is zero
    // too; the grouped form never reads them), the zero border of the V
    // image, the multiplicity table (the grouped form writes every entry of
    // its routing table)
    if constexpr (!G::GROUP) {
      for (int e = nkeys * 4 + tid; e < 32 * NKB2 * 4; e += NT) {
        *(uint4*)(Ks + e * 8) = make_uint4(0, 0, 0, 0);
        *(uint4*)(Vs + e * 8) = make_uint4(0, 0, 0, 0);
      }
    }
    for (int e = tid; e < HP * WP * 4; e += NT) {
      const int pc = fdiv(e, A.f_wp4);
      const int px = (e - pc * WP * 4) >> 2;
      if ((unsigned)(pc - P) >= (unsigned)H || (unsigned)(px - P) >= (unsigned)W)
        *(uint4*)(Vi + e * 8) = make_uint4(0, 0, 0, 0);
    }
    if constexpr (!G::GROUP)
      for (int e = tid; e < nqr * 4; e += NT) *(uint4*)(ct + e * 16) = make_uint4(0, 0, 0, 0);
    // per region (padded to whole query blocks, clamped into [0, R)): the
    // byte offset in the V image of its top-left pixel, with bit 5 carrying
    // the parity of its region column (the swizzle of its pixel pairs)
    for (int r = tid; r < 4 * A.nqb; r += NT) {
      const int rr = min(r, R - 1);
      const int ry = fdiv(rr, A.f_S), rx = rr - ry * S;
      rtab[r] = (2 * ry * WP + 2 * rx) * kHd * 2 + ((rx & 1) << 5);
    }
    __syncthreads();                                 // the table is clear before the counts
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      const int e = i * NT + tid;
      if (e < total) {
        const int p = e >> 2, g = e & 3;
        const int y = fdiv(p, A.f_W), x = p - y * W;
        const int ry = y >> 1, rx = x >> 1;
        const int pos = (ry * S + rx) * n + (y & 1) * 2 + (x & 1);
        *(uint4*)(Ks + pos * kHd + ((g ^ kswz(pos)) << 3)) = kr[i];
        if constexpr (G::GROUP)
          *(uint4*)(lds + G::VS_OFF + (g >> 1) * G::VH + pos * 32 + (g & 1) * 16) = vr[i];
        else
          *(uint4*)(Vs + pos * kHd + ((g ^ vrswz(pos)) << 3)) = vr[i];
        const int py = y + P, px = x + P;
        *(uint4*)(Vi + (py * WP + px) * kHd + ((g ^ vmswz(px)) << 3)) = vr[i];
      }
    }
    // LePE weights as bf16 pairs, per kernel row dy and pair kk: for the
    // even output column of a pair of columns the taps (w0,w1) (w2,w3)
    // (w4,0) over pixel pairs (x,x+1) (x+2,x+3) (x+4,x+5), for the odd
    // column (0,w0) (w1,w2) (w3,w4) over the same pairs
    if (we < KS * 3 * kHd) {
      const int kk = (we >> 5) % 3;
      wpr[we] = kk == 0 ? make_uint2(pack_bf16x2(wt[0], wt[1]), pack_bf16x2(0.f, wt[0]))
              : kk == 1 ? make_uint2(pack_bf16x2(wt[2], wt[3]), pack_bf16x2(wt[1], wt[2]))
                        : make_uint2(pack_bf16x2(wt[4], 0.f), pack_bf16x2(wt[3], wt[4]));
    }
    if constexpr (G::GROUP) {
      // routing tables: entry j = 4m + s of query region rl at int
      // rl * TOPK + s * KB + m, so the KB entries a lane needs (s = its
      // row's region slot) are contiguous.  K table: the byte offset of the
      // routed region's first K row, kr * 256, with the region's parity in
      // bit 5 (the parity part of the K rows' chunk swizzle); V table
      // (nqr * TOPK ints further): the byte offset of its first row in the
      // low V half-array (indices clamped into [0, R))
      int* tab = (int*)ct;
#pragma unroll
      for (int i = 0; i < NES; ++i) {
        const int e = i * NT + tid;
        if (e < nent) {
          const int kr = min(max(ent[i], 0), R - 1);
          const int rl = e / TOPK, j = e - rl * TOPK;
          const int o = rl * TOPK + (j & 3) * G::KB + (j >> 2);
          tab[o] = kr * 256 | ((kr & 1) << 5);
          tab[nent + o] = G::VS_OFF + kr * 128;
        }
      }
    } else {
      // multiplicities: routed key region kr of query region rl counts at
      // byte (kr % 4) * 16 + kr / 4 of row rl (indices clamped into [0, R));
      // byte counts stay below 256 (at most TOPK entries a row)
#pragma unroll
      for (int i = 0; i < NES; ++i) {
        const int e = i * NT + tid;
        if (e < nent) {
          const int kr = min(max(ent[i], 0), R - 1);
          const int slot = (kr & 3) * 16 + (kr >> 2);
          __atomic_fetch_add((uint32_t*)(ct + (e / TOPK) * 64 + (slot & ~3)),
                             1u << (8 * (slot & 3)), __ATOMIC_RELAXED);
        }
      }
    }
  }
  const float b0 = A.bias ? A.bias[c0 + cw] : 0.f;
  __syncthreads();

  const float c = A.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u, 0x3f803f80u));
  float* Lw = (float*)(lds + A.lw_off) + wave * 16 * LSW;
  const int grp = lane >> 5;                         // LePE: region row grp of each region
  // LePE transposing reads: lane i of a 16-lane row addresses padded pixel
  // x + i/4 (+4 for the second read) of row 2ry + grp + dy, channels
  // cq .. cq+3 with cq = (cw & ~15) + 4(i % 4), and receives channel cw of
  // the four pixels as two bf16 pairs along x.  The swizzle of pixel x + i/4
  // is bit 1 of it: the region column's parity (from the table) xor bit 3
  // of the lane.
  const int cq = (cw & ~15) + 4 * (lane & 3);
  const uint32_t lx = ((uint32_t)((lq >> 3) & 1) << 5) ^ ((uint32_t)(cq >> 3) << 4);
  const uint32_t lbase = (uint32_t)A.vi_off + (uint32_t)(grp * WP + (lq >> 2)) * kHd * 2 +
                         (uint32_t)(cq & 7) * 2;
  const uint32_t rs = (uint32_t)WP * kHd * 2;         // bytes per padded row
  // the previous block's output is stored once this block's logits are
  // under way, so the store's registers are not needed again at once
  uint4 pend_v = make_uint4(0, 0, 0, 0);
  uint32_t pend_off = kOob;
  for (; qb < qb1; qb += NW) {
    const bf16x8 qop = __builtin_bit_cast(bf16x8, qn);
    // the next block's Q, always issued (past the range it reads zeros) and
    // kept at the top of the block, so its latency hides behind the block
    qn = bload16(Qr, qb + NW < qb1 ? q_off(qb + NW) : kOob);
    __builtin_amdgcn_sched_barrier(0);
    const int qr = 4 * qb + (lq >> 2);
    // ---- LePE of the block's 16 pixels: region j's pixel row grp, two
    // columns, one kernel row dy a step (the grouped form spreads the rows
    // over the attention phases, to fill their latency) ----
    float lw[4][2];
    uint32_t va[4];
    {
      const int4 tb = *(const int4*)(rtab + 4 * qb);
      const int tj[4] = {tb.x, tb.y, tb.z, tb.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lw[j][0] = lw[j][1] = b0;
        va[j] = ((uint32_t)tj[j] ^ lx) + lbase;
      }
    }
    auto lepe_rows = [&](int dy0, int dy1) {
#pragma unroll
      for (int dy = 0; dy < KS; ++dy) {
        if (dy < dy0 || dy >= dy1) continue;
        const uint2 w0 = wpr[(dy * 3 + 0) * kHd + cw];
        const uint2 w1 = wpr[(dy * 3 + 1) * kHd + cw];
        const uint2 w2 = wpr[(dy * 3 + 2) * kHd + cw];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* pa = (const uint16_t*)(lds + va[j] + dy * rs);
          const uint2 a = lds_read_tr16(pa);
          const uint2 bb = lds_read_tr16(pa + 4 * kHd);
          lw[j][0] = dot2(w2.x, bb.x, dot2(w1.x, a.y, dot2(w0.x, a.x, lw[j][0])));
          lw[j][1] = dot2(w2.y, bb.x, dot2(w1.y, a.y, dot2(w0.y, a.x, lw[j][1])));
        }
      }
    };
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
    if constexpr (G::GROUP) {
      constexpr int KB = G::KB;
      const int* tab = (const int*)ct;
      const int own = lq >> 2;                        // this column's region of the block
      // routing rows of the block's four query regions (regions past R read
      // row R - 1; their outputs are not stored): the K entries of this
      // lane's key-row slot, the V entries of its transposing-read slot
      int tk[4][KB], tv[4][KB];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int* row = tab + (min(4 * qb + a, R - 1) - qr0) * TOPK;
#pragma unroll
        for (int m2 = 0; m2 < KB; ++m2) {
          tk[a][m2] = row[own * KB + m2];
          tv[a][m2] = row[nqr * TOPK + lg * KB + m2];
        }
      }
      // Q operands keeping only region a's columns
      const bf16x8 zero = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
      bf16x8 qa[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = own == a ? qop : zero;

      // ---- S^T: key block kb holds routed slots 4kb .. 4kb+3 of every
      // region; lane (lq, lg) supplies token lq % 4 of slot 4kb + lq / 4,
      // chunk lg (the K rows' swizzle: lg ^ (token >> 1) ^ 2 (parity)) ----
      const uint32_t tok = lq & 3;
      const uint32_t lck = tok * 64 + (((uint32_t)lg ^ (tok >> 1)) << 4);
      float x[KB][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const bf16x8 ka = *(const bf16x8*)(lds + ((uint32_t)tk[a][kb] ^ lck));
          sv = mfma_bf16(ka, qa[a], sv);
        }
        // lane holds token e of slot 4kb + lg, for its own region and query lq
#pragma unroll
        for (int e = 0; e < 4; ++e) x[kb][e] = sv[e];
      }
      __builtin_amdgcn_sched_barrier(0);
      lepe_rows(0, 2);
      __builtin_amdgcn_sched_barrier(0);
      bstore16(Or, pend_off, pend_v);
      float m = x[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, x[kb][e]);
      m = fmaxf(m, xor16(m));
      m = fmaxf(m, xor32(m));
      const float mc = m * c;

      // ---- numerators in P^T slot order (slots 0-3: slot 8h + lg, 4-7: slot
      // 8h + 4 + lg); O^T += V^T P^T per region, 32 keys a step ----
      uint32_t ph[2 * KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        ph[2 * kb] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(x[kb][0], c, -mc)),
                                 __builtin_amdgcn_exp2f(fmaf(x[kb][1], c, -mc)));
        ph[2 * kb + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(x[kb][2], c, -mc)),
                                     __builtin_amdgcn_exp2f(fmaf(x[kb][3], c, -mc)));
      }
      // V^T operands: lane (lq, lg) addresses token lq / 4 of slots 8h + lg
      // and 8h + 4 + lg, channels 4(lq % 4) .. +3 of each 16-channel half
      // (128 contiguous bytes for the 16 lanes of a row)
      const uint32_t lv = (lq >> 2) * 32 + (lq & 3) * 8;
      __builtin_amdgcn_sched_barrier(0);
      lepe_rows(2, 4);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < KB / 2; ++hh) {
        const bf16x8 phi = __builtin_bit_cast(
            bf16x8, make_uint4(ph[4 * hh], ph[4 * hh + 1], ph[4 * hh + 2], ph[4 * hh + 3]));
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const unsigned char* r0 = lds + ((uint32_t)tv[a][2 * hh] + lv);
          const unsigned char* r1 = lds + ((uint32_t)tv[a][2 * hh + 1] + lv);
          const uint2 a0 = lds_read_tr16((const uint16_t*)r0);
          const uint2 a1 = lds_read_tr16((const uint16_t*)r1);
          const uint2 d0 = lds_read_tr16((const uint16_t*)(r0 + G::VH));
          const uint2 d1 = lds_read_tr16((const uint16_t*)(r1 + G::VH));
          const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
          const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
          const bf16x8 pa = own == a ? phi : zero;
          acc0 = mfma_bf16(va, pa, acc0);
          acc1 = mfma_bf16(vb, pa, acc1);
          accl = mfma_bf16(ones, pa, accl);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      lepe_rows(4, KS);
    } else {
      const int cc = 4 * (lq & 3);
      const int ga = cc >> 3, gb = (16 + cc) >> 3, wi = cc & 7;
      const int qrl = min(qr, R - 1) - qr0;             // row of the multiplicity table
      // multiplicities of key regions 4 kb + lg, kb = 0..15, for this column
      const uint4 cnt = *(const uint4*)(ct + qrl * 64 + lg * 16);
      const uint32_t cw4[4] = {cnt.x, cnt.y, cnt.z, cnt.w};

      // ---- S^T = K Q^T over every key block; the largest routed logit ----
      float x[NKB][4];
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int pos = 16 * kb + lq;
        const bf16x8 ka = *(const bf16x8*)(Ks + pos * kHd + ((lg ^ kswz(pos)) << 3));
        const f32x4 sv = mfma_bf16(ka, qop, f32x4{0.f, 0.f, 0.f, 0.f});
  #pragma unroll
        for (int e = 0; e < 4; ++e) x[kb][e] = sv[e];
      }
      bstore16(Or, pend_off, pend_v);
      float m = -3.0e38f;
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bool routed = (cw4[kb >> 2] >> (8 * (kb & 3))) & 0xff;
        const float mk = fmaxf(fmaxf(x[kb][0], x[kb][1]), fmaxf(x[kb][2], x[kb][3]));
        m = routed ? fmaxf(m, mk) : m;
      }
      m = fmaxf(m, xor16(m));
      m = fmaxf(m, xor32(m));
      const float mc = m * c;

      // ---- numerators in P^T slot order; O^T += V^T P^T, 32 keys a step ----
  #pragma unroll
      for (int hh = 0; hh < NKB2; ++hh) {
        uint32_t ph[4];
  #pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kb = 2 * hh + half;
          const float cm = (float)((cw4[kb >> 2] >> (8 * (kb & 3))) & 0xff);
          float pv[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = cm * __builtin_amdgcn_exp2f(fmaf(x[kb][e], c, -mc));
          ph[2 * half] = pack_bf16x2(pv[0], pv[1]);
          ph[2 * half + 1] = pack_bf16x2(pv[2], pv[3]);
        }
        // V^T operands: lane (lq, lg) addresses key row 32hh + 4lg + lq/4 (+16),
        // channels 4(lq % 4) .. +3 of each 16-channel half, and receives
        // channel d0 + lq of rows 4lg + 0..3
        const int vrow = 32 * hh + 4 * lg + (lq >> 2);
        const uint16_t* r0p = Vs + vrow * kHd;
        const uint16_t* r1p = r0p + 16 * kHd;
        const int s0 = vrswz(vrow), s1 = vrswz(vrow + 16);
        const uint2 a0 = lds_read_tr16(r0p + ((ga ^ s0) << 3) + wi);
        const uint2 a1 = lds_read_tr16(r1p + ((ga ^ s1) << 3) + wi);
        const uint2 d0 = lds_read_tr16(r0p + ((gb ^ s0) << 3) + wi);
        const uint2 d1 = lds_read_tr16(r1p + ((gb ^ s1) << 3) + wi);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(d0.x, d0.y, d1.x, d1.y));
        const bf16x8 phi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
        acc0 = mfma_bf16(va, phi, acc0);
        acc1 = mfma_bf16(vb, phi, acc1);
        accl = mfma_bf16(ones, phi, accl);
      }
      lepe_rows(0, KS);
    }

#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kx = 0; kx < 2; ++kx) Lw[(j * 4 + grp * 2 + kx) * LSW + cw] = lw[j][kx];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- out = O / l + L, one rounding, 16-byte stores ----
    {
      const int t = lq & 3;
      const float inv = __builtin_amdgcn_rcpf(accl[0]);
      const float* lp = Lw + lq * LSW;
      const float4 a0 = *(const float4*)(lp + 4 * lg);
      const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
      const uint32_t o0x = pack_bf16x2(fmaf(acc0[0], inv, a0.x), fmaf(acc0[1], inv, a0.y));
      const uint32_t o0y = pack_bf16x2(fmaf(acc0[2], inv, a0.z), fmaf(acc0[3], inv, a0.w));
      const uint32_t o1x = pack_bf16x2(fmaf(acc1[0], inv, a1.x), fmaf(acc1[1], inv, a1.y));
      const uint32_t o1y = pack_bf16x2(fmaf(acc1[2], inv, a1.z), fmaf(acc1[3], inv, a1.w));
      const auto sx = __builtin_amdgcn_permlane16_swap(o0x, o1x, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(o0y, o1y, false, false);
      const bool odd = lg & 1;
      const uint4 ov = odd ? make_uint4(sx[0], sy[0], o1x, o1y) : make_uint4(o0x, o0y, sx[1], sy[1]);
      const int ch = odd ? 16 + 4 * (lg - 1) : 4 * lg;
      const int qrc = min(qr, R - 1);
      const int ry = fdiv(qrc, A.f_S), rx = qrc - ry * S;
      const uint32_t op = ((ry * 2 + (t >> 1)) * W + rx * 2 + (t & 1)) * C + c0 + ch;
      pend_off = qr < R ? op * 2 : kOob;
      pend_v = ov;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  bstore16(Or, pend_off, pend_v);
}

template <class G>
struct MaskLds {
  int ks_off, vs_off, vi_off, ct_off, rt_off, ws_off, lw_off;
  size_t bytes;
};

template <class G>
MaskLds<G> mask_lds(int H, int W, int nqr, int nqb) {
  MaskLds<G> l;
  const int WP = W + 2 * G::P, HP = H + 2 * G::P;
  const size_t rows = (size_t)G::NKB2 * 32;
  size_t off = 0;
  l.ks_off = (int)off;
  off += rows * kHd * 2;
  l.vs_off = (int)off;
  off += rows * kHd * 2;
  l.vi_off = (int)off;
  off += ((size_t)HP * WP + WP) * kHd * 2;
  l.ct_off = (int)off;
  off += (size_t)nqr * (G::GROUP ? 2 * G::TOPK * 4 : 64);   // K and V tables / multiplicities
  off = (off + 15) / 16 * 16;
  l.rt_off = (int)off;
  off += (size_t)nqb * 4 * 4;
  l.ws_off = (int)off;
  off += (size_t)G::KS * 3 * kHd * 8;
  l.lw_off = (int)off;
  off += (size_t)G::NW * 16 * G::LSW * 4;
  l.bytes = off;
  return l;
}

template <class G>
hipError_t mask_launch(MaskArgs a, hipStream_t st) {
  int dev = 0, lds_max = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (lds_max < 64 * 1024) lds_max = 64 * 1024;
  const void* fn = reinterpret_cast<const void*>(&attend_image_mask_kernel<G>);
  const MaskLds<G> l1 = mask_lds<G>(a.H, a.W, a.R, a.nqb);
  if (l1.bytes > (size_t)lds_max) return hipErrorNotSupported;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)l1.bytes);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_image_mask_kernel<G>, G::NT,
                                                   l1.bytes);
  if (e != hipSuccess) return e;
  // workgroups per (image, head): as many query-block ranges (1, 2 or 4) as
  // the resident workgroup slots take
  const long long slots = (long long)cus * (per_cu > 0 ? per_cu : 1);
  const long long base = (long long)a.B * a.heads;
  int qsplit = 1;
  while (qsplit < 4 && qsplit * 2 <= a.nqb && base * qsplit * 2 <= slots) qsplit *= 2;
  a.qsplit = qsplit;
  a.qper = (a.nqb + qsplit - 1) / qsplit;
  a.f_qsplit = make_fastdiv(qsplit);
  const MaskLds<G> l = mask_lds<G>(a.H, a.W, 4 * a.qper, a.nqb);
  a.ks_off = l.ks_off; a.vs_off = l.vs_off; a.vi_off = l.vi_off; a.ct_off = l.ct_off;
  a.rt_off = l.rt_off; a.ws_off = l.ws_off; a.lw_off = l.lw_off;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)l.bytes);
  if (e != hipSuccess) return e;
  const long long groups = (long long)(a.B + kXcds - 1) / kXcds * a.heads * qsplit * kXcds;
  if (groups >= (1LL << 31)) return hipErrorNotSupported;
  hipLaunchKernelGGL(attend_image_mask_kernel<G>, dim3((unsigned)groups), dim3(G::NT), l.bytes,
                     st, a);
  return hipGetLastError();
}

// LDS layout of one workgroup (bytes): K region-major [H*W][32] bf16, the
// padded V image [(H+2P)*(W+2P)][32] bf16 (plus one row of slack for the
// LePE reads past the last tap), the routing table [rper][topk] int2 and
// the wavefronts' L tiles.
template <class G>
struct ImageLds {
  int ks_off, vs_off, it_off, lw_off, wt_off;
  size_t bytes;
};

template <class G>
ImageLds<G> image_lds(int H, int W, int rper) {
  ImageLds<G> l;
  const int WP = W + 2 * G::P, HP = H + 2 * G::P;
  size_t off = 0;
  l.ks_off = (int)off;
  off += (size_t)H * W * kHd * 2;
  l.vs_off = (int)off;
  off += ((size_t)HP * WP + WP) * kHd * 2;
  l.it_off = (int)off;
  off += (size_t)rper * G::TOPK * 8;
  off = (off + 15) / 16 * 16;
  l.lw_off = (int)off;
  off += (size_t)G::NW * 16 * G::LSW * 4;
  l.wt_off = (int)off;
  off += (size_t)G::KK * kHd * 4;
  l.bytes = off;
  return l;
}

template <class G>
hipError_t image_launch(ImageArgs a, int rsplit, hipStream_t st) {
  int dev = 0, lds_max = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (lds_max < 64 * 1024) lds_max = 64 * 1024;
  const void* fn = reinterpret_cast<const void*>(&attend_image_kernel<G>);
  // workgroups per (image, head): 1, 2 or 4 ranges of query regions, as
  // many as the resident workgroup slots take (the smaller batches)
  if (rsplit < 1) {
    const ImageLds<G> l1 = image_lds<G>(a.H, a.W, a.R);
    if (l1.bytes > (size_t)lds_max) return hipErrorNotSupported;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)l1.bytes);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_image_kernel<G>, G::NT,
                                                     l1.bytes);
    if (e != hipSuccess) return e;
    const long long slots = (long long)cus * (per_cu > 0 ? per_cu : 1);
    const long long base = (long long)a.B * a.heads;
    rsplit = 1;
    while (rsplit < 4 && rsplit * 2 <= a.R && base * rsplit * 2 <= slots) rsplit *= 2;
  }
  if (rsplit > a.R) rsplit = a.R;
  a.rsplit = rsplit;
  a.rper = (a.R + rsplit - 1) / rsplit;
  a.f_rsplit = make_fastdiv(rsplit);
  const ImageLds<G> l = image_lds<G>(a.H, a.W, a.rper);
  if (l.bytes > (size_t)lds_max) return hipErrorNotSupported;
  a.ks_off = l.ks_off; a.vs_off = l.vs_off; a.it_off = l.it_off; a.lw_off = l.lw_off;
  a.wt_off = l.wt_off;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)l.bytes);
  if (e != hipSuccess) return e;
  const long long groups = (long long)(a.B + kXcds - 1) / kXcds * a.heads * a.rsplit * kXcds;
  if (groups >= (1LL << 31)) return hipErrorNotSupported;
  hipLaunchKernelGGL(attend_image_kernel<G>, dim3((unsigned)groups), dim3(G::NT), l.bytes, st, a);
  return hipGetLastError();
}

// 4x4-pixel regions (a 28x28 map's padded image of one head is 66 KB): 16
// wavefronts, one workgroup a CU; 2x2-pixel regions (14x14: 22 KB): 8
// wavefronts, two workgroups a CU
#ifndef BRA_IMAGE_NW2
#define BRA_IMAGE_NW2 16
#endif
#ifndef BRA_IMAGE_NW3
#define BRA_IMAGE_NW3 8
#endif
using ImgSt2 = Ic<4, 4, 4, 5, BRA_IMAGE_NW2>;
using ImgSt3 = Ic<2, 2, 16, 5, BRA_IMAGE_NW3>;
// 4x4 regions with top-2 or top-8 (32 or 128 routed keys; top-16 would
// spill at sixteen wavefronts a workgroup)
template <int TOPK>
using Img4 = Ic<4, 4, TOPK, 5, BRA_IMAGE_NW2>;
#ifndef BRA_MASK_NW
#define BRA_MASK_NW 8
#endif
template <int NKB2>
using MaskSt3 = Im<16, BRA_MASK_NW, NKB2>;
template <int NKB2>
using GroupSt3 = Im<16, BRA_MASK_NW, NKB2, true>;

}  // namespace

#ifndef BRA_IMAGE_RSPLIT
#define BRA_IMAGE_RSPLIT 0
#endif

hipError_t launch_attend_image(const void* q, const void* k, const void* v, const int32_t* idx,
                               const Shape& s, float attn_scale, const float* w,
                               const float* bias, int ks, void* out, hipStream_t st) {
  if (!w || ks != 5 || s.C != s.heads * kHd || s.Hf != s.H) return hipErrorNotSupported;
  if ((long long)s.H * s.W * s.C * 2 >= (long long)kOob) return hipErrorNotSupported;
  if (s.H + 4 >= (1 << 15) || s.W + 4 >= (1 << 15)) return hipErrorNotSupported;
  ImageArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.idx = idx; a.out = (uint16_t*)out; a.w = w; a.bias = bias;
  a.B = s.B; a.H = s.H; a.W = s.W; a.C = s.C; a.S = s.S; a.R = s.R; a.heads = s.heads;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.f_S = make_fastdiv(s.S);
  a.f_W = make_fastdiv(s.W);
  a.f_heads = make_fastdiv(s.heads);
  a.f_wp4 = make_fastdiv((s.W + 4) * 4);
  const int rsplit = BRA_IMAGE_RSPLIT;                // 0: chosen from the batch
  auto is = [&](int hs, int ws, int topk) { return s.hs == hs && s.ws == ws && s.topk == topk; };
  // 2x2 regions, up to 64 of them: the grouped form (a query's softmax over
  // its 4 topk routed keys) unless the image holds no more keys than that
  // in whole 32-key steps, where the masked form (every key of the image,
  // one MFMA per 16 keys, no per-region selects) is the cheaper one
  if (s.hs == 2 && s.ws == 2 && s.topk == MaskSt3<1>::TOPK && s.R <= 64) {
    MaskArgs m;
    m.q = a.q; m.k = a.k; m.v = a.v; m.idx = a.idx; m.out = a.out; m.w = a.w; m.bias = a.bias;
    m.B = s.B; m.H = s.H; m.W = s.W; m.C = s.C; m.S = s.S; m.R = s.R; m.heads = s.heads;
    m.nqb = (s.R + 3) / 4;
    m.nkb = (s.R * 4 + 15) / 16;
    m.scale_log2 = a.scale_log2;
    m.f_S = a.f_S; m.f_W = a.f_W; m.f_heads = a.f_heads; m.f_wp4 = a.f_wp4;
    hipError_t e = hipErrorNotSupported;
    switch ((s.R * 4 + 31) / 32) {          // 32-key steps of the image
      case 2: e = mask_launch<MaskSt3<2>>(m, st); break;
      case 3: e = mask_launch<GroupSt3<3>>(m, st); break;
      case 4: e = mask_launch<GroupSt3<4>>(m, st); break;
      case 5: e = mask_launch<GroupSt3<5>>(m, st); break;
      case 6: e = mask_launch<GroupSt3<6>>(m, st); break;
      case 7: e = mask_launch<GroupSt3<7>>(m, st); break;
      case 8: e = mask_launch<GroupSt3<8>>(m, st); break;
      default: break;
    }
    if (e != hipErrorNotSupported) return e;
  }
  if (is(ImgSt2::HS, ImgSt2::WS, ImgSt2::TOPK)) return image_launch<ImgSt2>(a, rsplit, st);
  if (is(4, 4, 2)) return image_launch<Img4<2>>(a, rsplit, st);
  if (is(4, 4, 8)) return image_launch<Img4<8>>(a, rsplit, st);
  if (is(ImgSt3::HS, ImgSt3::WS, ImgSt3::TOPK)) return image_launch<ImgSt3>(a, rsplit, st);
  return hipErrorNotSupported;
}

}  // namespace bra
