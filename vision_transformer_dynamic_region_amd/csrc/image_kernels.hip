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
//   LePE       5x5 cross-correlation of the padded V image in float32 FMAs
//              (the float32 weights as given, the bf16 pixels widened
//              exactly), interleaved with the attention phases;
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
  static constexpr int NB = 8;                         // staging vectors in flight a thread
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
  int ks_off, vs_off, it_off, lw_off;   // LDS byte offsets
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
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
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

  // ---- stage: K region-major, V into the padded image, routing rows ----
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
    // the zero border of the V image (position within a pixel does not matter)
    for (int e = tid; e < HP * WP * 4; e += NT) {
      const int pc = fdiv(e, A.f_wp4);               // padded row
      const int px = (e - pc * WP * 4) >> 2;
      if ((unsigned)(pc - P) >= (unsigned)H || (unsigned)(px - P) >= (unsigned)W)
        *(uint4*)(Vs + e * 8) = make_uint4(0, 0, 0, 0);
    }
    // routing rows of this workgroup's query regions: the routed region's
    // first key position and the padded image coordinates of its top-left
    // pixel (indices clamped into [0, R))
    for (int e = tid; e < (r1 - r0) * TOPK; e += NT) {
      const int reg = min(max(A.idx[((size_t)b * A.R + r0) * TOPK + e], 0), A.R - 1);
      const int sy = fdiv(reg, A.f_S), sx = reg - sy * S;
      itab[e] = make_int2(reg * n, ((sy * HS + P) << 16) | (sx * WS + P));
    }
  }

  // this channel lane's LePE weights, float32 as given
  const int cw = lane & 31;
  float wf[KS][KS];
  {
    const float* wp = A.w + (size_t)(c0 + cw) * KK;
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
      for (int jx = 0; jx < KS; ++jx) wf[i][jx] = wp[i * KS + jx];
  }
  const float b0 = A.bias ? A.bias[c0 + cw] : 0.f;
  __syncthreads();

  const float c = A.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u, 0x3f803f80u));
  float* Lw = (float*)(lds + A.lw_off) + wave * 16 * LSW;   // this wavefront's L tile
  const int grp = lane >> 5;
  const int xw = (grp % NXG) * XG, yl = (grp / NXG) * TYW;

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
  uint4 qn = bload16(Qr, task < ntask ? q_off(task) : kOob);
  for (; task < ntask; task += NW) {
    const bf16x8 qop = __builtin_bit_cast(bf16x8, qn);
    if (task + NW < ntask) qn = bload16(Qr, q_off(task + NW));
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
    // four pixels as two bf16 pairs along x; the taps are float32 FMAs on
    // the widened pixels
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
        // pixels x .. x+7 of this tap row (x+6, x+7 unused when XG == 2)
        const float f[8] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y),
                            bf16_lo(bb.x), bf16_hi(bb.x), bf16_lo(bb.y), bf16_hi(bb.y)};
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const int rr = dy - i;
          if (rr < 0 || rr >= TYW) continue;
#pragma unroll
          for (int kx = 0; kx < XG; ++kx)
#pragma unroll
            for (int jx = 0; jx < KS; ++jx) lw[rr][kx] = fmaf(wf[i][jx], f[kx + jx], lw[rr][kx]);
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

// LDS layout of one workgroup (bytes): K region-major [H*W][32] bf16, the
// padded V image [(H+2P)*(W+2P)][32] bf16 (plus one row of slack for the
// LePE reads past the last tap), the routing table [rper][topk] int2 and
// the wavefronts' L tiles.
template <class G>
struct ImageLds {
  int ks_off, vs_off, it_off, lw_off;
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
  if (is(ImgSt2::HS, ImgSt2::WS, ImgSt2::TOPK)) return image_launch<ImgSt2>(a, rsplit, st);
  if (is(ImgSt3::HS, ImgSt3::WS, ImgSt3::TOPK)) return image_launch<ImgSt3>(a, rsplit, st);
  return hipErrorNotSupported;
}

}  // namespace bra
