// Fused gather-attention + LePE for bf16 inputs whose region shape is known at
// compile time (the BiFormer stage shapes and the 512^2 segmentation shape):
// one persistent, software-pipelined kernel per shape.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3: gather of the routed regions' tokens, softmax attention, LePE added to
// the output), p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉
// Transformer的计算范式" (§4: the depthwise LePE conv on V), p5 = hyper.ai
// abstract of BiFormer (token-to-token attention over the union of the routed
// regions).
//
// Work split.  A unit is (image, query region, block of CB channels = CB/32
// heads) and has exactly four tasks (16-query block x head), one per
// wavefront.  The units of an XCD are dealt round-robin to that XCD's
// workgroups, so at any moment one XCD works on neighbouring regions of one
// image and its L2 serves their shared halo rows and routed regions.  Per
// unit:
//   1. commit: the unit's V halo (region plus 2 pixels each side, zero
//      outside the image; bf16 as loaded), the routed regions' K and V rows
//      (row-major, 16-byte chunks XOR-swizzled by row) go from registers to
//      LDS; barrier;
//   2. the global loads of the next unit (query operands, routed K/V vectors,
//      halo) are issued into registers;
//   3. each wavefront, on its own task only:
//      attention  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (one query per lane
//                 column), softmax numerators in float32 with the scale
//                 folded into exp2, rounded to bf16; O^T = V^T P^T with the
//                 V^T operands read straight from the row-major V tile by the
//                 transposing LDS read; the row sums by one more MFMA against
//                 a ones operand (so O is normalised by exactly the weights
//                 it was built from);
//      LePE       the wavefront's own 16 pixels x 32 channels: 5x5
//                 cross-correlation on v_dot2_f32_bf16 (tap pairs along x,
//                 weights rounded once to bf16, products exact, float32
//                 accumulation), four halo pixels of a channel fetched per
//                 transposing LDS read; the two are interleaved phase by
//                 phase so the convolution fills the MFMA/softmax latency;
//      epilogue   L through a wavefront-private LDS tile into the MFMA
//                 layout, out = O / l + L rounded once to bf16, 16-byte
//                 stores;
//   4. with one staging buffer, a barrier before the next commit; with two
//      (DB), none: the next unit stages into the other buffer.
// Nothing but the output is written to memory: the gathered K/V exist only
// in LDS.

#include "device_common.h"
#include "launch_plan.h"

namespace bra {
namespace {

constexpr int kHd = 32;    // head width

template <int C_, int CB_, int HS_, int WS_, int TOPK_, int KS_, bool DB_, int OCC_ = 2,
          bool NT_ = false, bool XP_ = false>
struct Rc {
  static constexpr int C = C_, CB = CB_, HS = HS_, WS = WS_, TOPK = TOPK_, KS = KS_;
  static constexpr bool DB = DB_;                  // double-buffered staging
  // Q, K and V projected from x in the kernel (the module's fused form): x
  // of the unit's queries, routed keys and halo pixels is loaded in the MFMA
  // operand layout and multiplied by the unit block's rows of Wq, Wk, Wv
  static constexpr bool XP = XP_;
  // more than 128 routed keys: S^T is not held in 4 KC / 64 registers but
  // taken 64 keys a step with a running maximum (the accumulators rescaled
  // when it grows; BRA_TWO_PASS: computed twice instead, the maximum first,
  // then the numerators 32 keys a step)
  static constexpr bool TWO_PASS = TOPK_ * HS_ * WS_ > 128;
#ifndef BRA_TWO_PASS
  static constexpr bool ONLINE = TWO_PASS;
#else
  static constexpr bool ONLINE = false;
#endif
  static constexpr int OCC = OCC_;                 // workgroups per CU to allow for
  // output stores non-temporal (written through, so the end-of-kernel
  // write-back is short; each 16-byte store then costs more HBM writes)
  static constexpr int OUT_CPOL = NT_ ? BRA_OUT_CPOL : 0;
  static constexpr int NCB = C / CB;               // channel blocks per region
  static constexpr int n = HS * WS;                // queries per region
  static constexpr int KC = TOPK * n;              // routed keys, all in LDS at once
  static constexpr int NQB = (n + 15) / 16;        // 16-query blocks
  static constexpr int HB = CB / kHd;              // heads per unit
  static constexpr int TASKS = NQB * HB;
  static constexpr int P = KS / 2;
  static constexpr int KK = KS * KS;
  static constexpr int HH = HS + KS - 1, HW = WS + KS - 1;
  static constexpr int GB = CB / 8;                // 16-byte vectors per pixel
  static constexpr int PSTEP = kThreads / GB;      // pixels per staging pass
  static constexpr int HPT = (HH * HW + PSTEP - 1) / PSTEP;
  static constexpr int KPT = (KC + PSTEP - 1) / PSTEP;
  // LePE items of a wavefront: 32 channels x the block's pixels, two items
  // per channel lane, each XG columns (tap pairs along x) by TYW rows
  static constexpr int QR = (n < 16 ? n : 16) / WS;      // pixel rows of a query block
  static constexpr int XG = WS % 4 == 0 ? 4 : WS;
  static constexpr int NXG = WS / XG;
  static constexpr int TYW = QR * NXG / 2;
  static constexpr int LSW = kHd + 4;               // wavefront L tile row stride (floats)
  // LDS: [halo | K | V] x (DB ? 2 : 1), wavefront L tiles, (XP) the unit
  // block's Wq, Wk and Wv rows and biases, routing table
  static constexpr int HALO = HH * HW * CB * 2;
  static constexpr int KVB = KC * CB * 2;
  static constexpr int BUF = (HALO + 2 * KVB + 15) / 16 * 16;
  static constexpr int L_OFF = BUF * (DB ? 2 : 1);
  static constexpr int WX_OFF = L_OFF + kWaves * 16 * LSW * 4;
  static constexpr int WX_BYTES = XP ? 3 * CB * C * 2 + 3 * CB * 4 : 0;
  static constexpr int NHB = (HH * HW + 15) / 16;  // (XP) 16-pixel blocks of the halo
  static constexpr int HBW = (NHB + kWaves - 1) / kWaves;   // halo blocks a wavefront
  static constexpr int IT_OFF = WX_OFF + WX_BYTES;

  static_assert(C % CB == 0 && CB % kHd == 0, "channel blocking");
  static_assert(TASKS == kWaves, "one task (16 queries x 1 head) per wavefront");
  static_assert(n >= 16 ? 16 % WS == 0 : n % WS == 0, "query blocks are whole pixel rows");
  static_assert(kThreads % GB == 0, "a thread stages one fixed 16-byte vector of a pixel");
  static_assert(KC % 32 == 0 && KC <= 256, "routed keys: a multiple of 32, one softmax step");
  static_assert(KS == 5 && (XG == 4 || XG == 2) && TYW >= 1 && (QR * NXG) % 2 == 0,
                "dot2 LePE: 5x5 taps, two items per channel lane");
  static_assert(KK * CB * 4 <= BUF, "weights are staged through the first buffer");
  static_assert(!XP || (C == 64 && n == 64 && KC == 16 * kWaves && !DB && HH * HW % 16 == 0),
                "fused projection: 64 channels of x, 8x8 regions, top-1, one buffer");
  static_assert(!XP || 16 * CB * 2 <= 16 * LSW * 4, "a wavefront's Q tile fits its L tile");
};

// Weight-row swizzle (XP): 16-byte chunk c (of eight) of row r sits at
// chunk c ^ ((r >> 1) & 7), so the 16 rows one operand load reads (8 even,
// 8 odd, 128 bytes apart) fall into 16 distinct bank groups.
__device__ __forceinline__ int xswz(int p) { return (p >> 1) & 7; }

// K/V tile swizzle: chunk g (16 bytes) of key row kk sits at chunk
// g ^ kswz(kk), so the 16 rows one operand load reads fall into 16 distinct
// bank groups.  kswz(kk + 16m) == kswz(kk).
template <int GB>
__device__ __forceinline__ int kswz(int kk) {
  if constexpr (GB >= 16) return kk & 15;
  else if constexpr (GB == 8) return (kk >> 1) & 7;
  else return (kk >> 2) & 3;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane
// row, lane j receives element j % 4 of the four 16-bit elements addressed by
// lanes j / 4 + 4e, e = 0..3 (as element e).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

struct RegionArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  const float* w;       // [C, KS, KS]
  const float* bias;    // [C] or null
  // XP: q, k and v point to x; wq, wk, wv to the C rows of Wq, Wk and Wv
  // ([C, C] bf16 each, rows = output channels) and bq, bk, bv to their
  // biases (or null)
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  const float* bq;
  const float* bk;
  const float* bv;
  int H, W, S, R;
  int Hf;               // rows of one frame; the LePE halo stays inside it
  float scale_log2;     // attn_scale * log2(e)
  int units;            // B * R * NCB
  int per_xcd;          // units per XCD (a multiple of NCB)
  int bpx;              // workgroups per XCD (a multiple of NCB)
  FastDiv f_R, f_S, f_syf;   // f_syf: region rows per frame
};

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer access to one image: loads at an offset past the end return
// zeros and stores there are dropped, so padding and masked lanes need no
// branches (and the wait counters stay exact across the pipelined loop).
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
template <int CPOL>
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, CPOL);
}

#ifndef BRA_PRIO_RAMP
#define BRA_PRIO_RAMP 1
#endif

template <class G>
__global__ __launch_bounds__(kThreads, G::OCC) void attend_region_kernel(RegionArgs A) {
  constexpr int C = G::C, CB = G::CB, HS = G::HS, WS = G::WS, TOPK = G::TOPK;
  constexpr int n = G::n, KC = G::KC, NQB = G::NQB, NCB = G::NCB;
  constexpr int P = G::P, KS = G::KS, KK = G::KK, HH = G::HH, HW = G::HW, GB = G::GB;
  constexpr int PSTEP = G::PSTEP, HPT = G::HPT, KPT = G::KPT;
  constexpr int XG = G::XG, NXG = G::NXG, TYW = G::TYW, LSW = G::LSW;
  extern __shared__ __align__(16) unsigned char lds[];
  int* itab = (int*)(lds + G::IT_OFF);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int u0 = xcd * A.per_xcd + slot;
  const int uend = min((xcd + 1) * A.per_xcd, A.units);
  if (u0 >= uend) return;                          // uniform over the workgroup
  const int nu = (uend - u0 + A.bpx - 1) / A.bpx;
  const int cb0 = (u0 % NCB) * CB;                 // same for every unit of this workgroup

  // routing rows of all this workgroup's units -> element offsets of the
  // routed regions' top-left pixels (indices clamped into [0, R))
  for (int e = tid; e < nu * TOPK; e += kThreads) {
    const int j = e / TOPK, t = e - j * TOPK;
    const int br = (u0 + j * A.bpx) / NCB;
    const int reg = min(max(A.idx[(size_t)br * TOPK + t], 0), A.R - 1);
    const int sy = fdiv(reg, A.f_S), sx = reg - sy * A.S;
    itab[e] = (sy * HS * A.W + sx * WS) * C;
  }
  // this block's LePE weights, transposed to [tap][channel] in the first
  // buffer (consecutive threads write consecutive LDS words)
  {
    float* wst = (float*)lds;
    for (int e = tid; e < KK * CB; e += kThreads) {
      const int t = e / CB, c = e - t * CB;
      wst[e] = A.w[(size_t)(cb0 + c) * KK + t];
    }
  }
  if constexpr (G::XP) {
    // the unit block's rows of Wq, Wk and Wv (swizzled) and their biases
    uint16_t* wqs = (uint16_t*)(lds + G::WX_OFF);
    uint16_t* wks = wqs + CB * C;
    uint16_t* wvs = wks + CB * C;
    float* bqs = (float*)(wvs + CB * C);
    float* bks = bqs + CB;
    float* bvs = bks + CB;
    for (int e = tid; e < CB * (C / 8); e += kThreads) {
      const int r = e / (C / 8), c = e - r * (C / 8);
      const int o = r * C + ((c ^ xswz(r)) * 8);
      *(uint4*)(wqs + o) = *(const uint4*)(A.wq + (size_t)(cb0 + r) * C + c * 8);
      *(uint4*)(wks + o) = *(const uint4*)(A.wk + (size_t)(cb0 + r) * C + c * 8);
      *(uint4*)(wvs + o) = *(const uint4*)(A.wv + (size_t)(cb0 + r) * C + c * 8);
    }
    for (int c = tid; c < CB; c += kThreads) {
      bqs[c] = A.bq ? A.bq[cb0 + c] : 0.f;
      bks[c] = A.bk ? A.bk[cb0 + c] : 0.f;
      bvs[c] = A.bv ? A.bv[cb0 + c] : 0.f;
    }
  }
  __syncthreads();

  // this wavefront's task: query block qb of head hb
  const int qb = wave % NQB, hb = wave / NQB;
  const int qrow0 = qb * 16 / WS;                  // first pixel row of the block
  // LePE items: channel cw (of the unit's block) of head hb, columns
  // xw .. xw+XG-1, block rows yl .. yl+TYW-1
  const int grp = lane >> 5;
  const int cw = hb * kHd + (lane & 31);
  const int xw = (grp % NXG) * XG, yl = (grp / NXG) * TYW;
  // dot2 weights per kernel row i: for an even output column the tap pairs
  // (w0,w1) (w2,w3) (w4,0) over input pairs (x,x+1) (x+2,x+3) (x+4,x+5); for
  // the odd column after it (0,w0) (w1,w2) (w3,w4) over the same pairs
  uint32_t we[KS][3], wo[KS][3];
  {
    const float* wst = (const float*)lds;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      float t[5];
#pragma unroll
      for (int jx = 0; jx < 5; ++jx) t[jx] = wst[(i * KS + jx) * CB + cw];
      we[i][0] = pack_bf16x2(t[0], t[1]);
      we[i][1] = pack_bf16x2(t[2], t[3]);
      we[i][2] = pack_bf16x2(t[4], 0.f);
      wo[i][0] = pack_bf16x2(0.f, t[0]);
      wo[i][1] = pack_bf16x2(t[1], t[2]);
      wo[i][2] = pack_bf16x2(t[3], t[4]);
    }
  }
  const float b0 = A.bias ? A.bias[cb0 + cw] : 0.f;

  const int g = tid % GB, pk = tid / GB;           // staged vector: pixel pk + PSTEP*i, chunk g
  auto decode = [&](int j, int& b, int& ry, int& rx) {
    const int br = (u0 + j * A.bpx) / NCB;
    b = fdiv(br, A.f_R);
    const int r = br - b * A.R;
    ry = fdiv(r, A.f_S);
    rx = r - ry * A.S;
  };

  const uint32_t img_elems = (uint32_t)A.H * A.W * C;
  const int q = qb * 16 + lq;                      // this lane's query (column of the MFMAs)
  // (array sizes of the unused form: 1)
  constexpr int KPA = G::XP ? 1 : KPT, HPA = G::XP ? 1 : HPT, HBA = G::XP ? G::HBW : 1;
  uint4 qn, kn[KPA], vn[KPA], hn[HPA];
  uint4 xqn[2], xkn[2], xhn[HBA][2];               // XP: x operands, k-steps 0 and 1
  uint32_t hok = 0;                                // XP: bit i: halo block i's pixel is in the image
  auto prefetch = [&](int j) {
    int b, ry, rx;
    decode(j, b, ry, rx);
    const size_t img = (size_t)b * img_elems;
    const auto Q = image_rsrc(A.q + img, img_elems * 2);
    const auto K = image_rsrc(A.k + img, img_elems * 2);
    const auto V = image_rsrc(A.v + img, img_elems * 2);
    if constexpr (G::XP) {
      // x in the projections' operand layout: lane (lq, lg) takes channels
      // 32s + 8lg .. +7 of this wavefront's query lq and of routed key
      // 16 wave + lq
      const int key = 16 * wave + lq;
      const uint32_t oq = ((ry * HS + q / WS) * A.W + rx * WS + q % WS) * C + 8 * lg;
      const uint32_t ok = itab[j * TOPK] + ((key / WS) * A.W + key % WS) * C + 8 * lg;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        xqn[s2] = bload16(Q, (oq + 32 * s2) * 2);
        xkn[s2] = bload16(K, (ok + 32 * s2) * 2);
      }
      // halo blocks wave, wave + 4, ...: pixel 16 blk + lq of the 12 x 12
      // halo (zero outside the image, as the V halo of the plain form)
      const int ftop = (int)fdiv(ry, A.f_syf) * A.Hf;
      hok = 0;
#pragma unroll
      for (int i = 0; i < G::HBW; ++i) {
        const int blk = wave + kWaves * i;
        const int pix = 16 * blk + lq;
        const int hy = pix / HW, hx = pix % HW;
        const int y = ry * HS - P + hy, x = rx * WS - P + hx;
        const bool in = (blk < G::NHB) & ((unsigned)(y - ftop) < (unsigned)A.Hf) &
                        ((unsigned)x < (unsigned)A.W);
        hok |= (in ? 1u : 0u) << i;
        const uint32_t oh = (uint32_t)((__umul24(y, A.W) + x) * C + 8 * lg);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) xhn[i][s2] = bload16(V, in ? (oh + 32 * s2) * 2 : kOob);
      }
    } else {
      const uint32_t off = ((ry * HS + q / WS) * A.W + rx * WS + q % WS) * C + cb0 + hb * kHd + 8 * lg;
      qn = bload16(Q, q < n ? off * 2 : kOob);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int kk = pk + PSTEP * i;               // pk < PSTEP
      const int tj = kk / n, tok = kk % n;
      const uint32_t off =
          (PSTEP * (i + 1) <= KC || kk < KC)
              ? (itab[j * TOPK + tj] + ((tok / WS) * A.W + tok % WS) * C + cb0 + g * 8) * 2
              : kOob;
      if constexpr (!G::XP) {
        kn[i] = bload16(K, off);
        vn[i] = bload16(V, off);
      }
    }
    if constexpr (G::XP) return;
    const int ftop = (int)fdiv(ry, A.f_syf) * A.Hf;  // first row of the region's frame
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int pix = pk + PSTEP * i;
      const int hy = pix / HW, hx = pix % HW;
      const int y = ry * HS - P + hy, x = rx * WS - P + hx;
      // one unsigned compare per bound; & rather than && keeps this branch-free
      const bool ok = (PSTEP * (i + 1) <= HH * HW || pix < HH * HW) &
                      ((unsigned)(y - ftop) < (unsigned)A.Hf) & ((unsigned)x < (unsigned)A.W);
      hn[i] = bload16(V, ok ? (uint32_t)((__umul24(y, A.W) + x) * C + cb0 + g * 8) * 2 : kOob);
    }
  };

  bf16x8 qop;
  auto commit = [&](unsigned char* buf) {
    uint16_t* Hs = (uint16_t*)buf;
    uint16_t* Ks = (uint16_t*)(buf + G::HALO);
    uint16_t* Vs = (uint16_t*)(buf + G::HALO + G::KVB);
    if constexpr (!G::XP) {
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int pix = pk + PSTEP * i;
        if (PSTEP * (i + 1) <= HH * HW || pix < HH * HW) *(uint4*)(Hs + pix * CB + g * 8) = hn[i];
      }
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int kk = pk + PSTEP * i;
        if (PSTEP * (i + 1) <= KC || kk < KC) {
          const int o = kk * CB + ((g ^ kswz<GB>(kk)) * 8);
          *(uint4*)(Ks + o) = kn[i];
          *(uint4*)(Vs + o) = vn[i];
        }
      }
      qop = __builtin_bit_cast(bf16x8, qn);
    }
  };

  const float c = A.scale_log2;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u,
                                                            0x3f803f80u, 0x3f803f80u));
  float* Lw = (float*)(lds + G::L_OFF) + wave * 16 * LSW;   // this wavefront's L tile
  prefetch(0);
  __syncthreads();                                  // weights read; the first buffer is free

  for (int j = 0; j < nu; ++j) {
    unsigned char* buf = lds + (G::DB ? (j & 1) * G::BUF : 0);
#if BRA_PRIO_RAMP
    {
      // waves further through their units issue at a lower priority, so the
      // workgroups sharing a CU (older ones are otherwise issued first) keep
      // pace and finish together
      const int lvl = __builtin_amdgcn_readfirstlane(4 * j / nu);
      if (lvl == 0) __builtin_amdgcn_s_setprio(3);
      else if (lvl == 1) __builtin_amdgcn_s_setprio(2);
      else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#endif
    commit(buf);
    if constexpr (G::XP) {
      // ---- before the barrier that publishes the staged tiles, and before
      // the next unit's loads reuse the x registers: K of the routed keys
      // (key block = wavefront) and this wavefront's Q: (Wq|Wk)[rows] x^T on v_mfma_f32_16x16x32_bf16 with the
      // bias added and one rounding to bf16, as the plain projection ----
      const uint16_t* wqs = (const uint16_t*)(lds + G::WX_OFF);
      const uint16_t* wks = wqs + CB * C;
      const uint16_t* wvs = wks + CB * C;
      const float* bqs = (const float*)(wvs + CB * C);
      const float* bks = bqs + CB;
      const float* bvs = bks + CB;
      uint16_t* Hw = (uint16_t*)buf;
      uint16_t* Kw = (uint16_t*)(buf + G::HALO);
      uint16_t* Vw = (uint16_t*)(buf + G::HALO + G::KVB);
      // weight row r(i) feeds D row i; D lane (lq, lg) holds the channels
      // r(4lg .. 4lg+3) of the operand's pixel lq, biased and rounded
      auto project = [&](const uint4* xo, const uint16_t* ws, const float* bs,
                         auto row) -> uint2 {
        const int r = row(lq);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < C / 32; ++s2) {
          const int c = 4 * s2 + lg;
          const bf16x8 wa = *(const bf16x8*)(ws + r * C + ((c ^ xswz(r)) * 8));
          acc = mfma_bf16(wa, __builtin_bit_cast(bf16x8, xo[s2]), acc);
        }
        const float4 bb = *(const float4*)(bs + row(4 * lg));   // r(4lg + e) = r(4lg) + e
        return make_uint2(pack_bf16x2(acc[0] + bb.x, acc[1] + bb.y),
                          pack_bf16x2(acc[2] + bb.z, acc[3] + bb.w));
      };
      {
        const int key = 16 * wave + lq;              // key block = wavefront
#pragma unroll
        for (int cb = 0; cb < CB / 16; ++cb) {
          const auto rows = [&](int i) { return 16 * cb + i; };
          const int ch = 2 * cb + (lg >> 1);         // 16-byte chunk of channels 16cb + 4lg
          const int o = key * CB + ((ch ^ kswz<GB>(key)) * 8) + 4 * (lg & 1);
          *(uint2*)(Kw + o) = project(xkn, wks, bks, rows);
          *(uint2*)(Vw + o) = project(xkn, wvs, bvs, rows);
        }
      }
      // V of the halo blocks (row-major [pixel][CB], zero outside the image)
#pragma unroll
      for (int i = 0; i < G::HBW; ++i) {
        const int blk = wave + kWaves * i;
        if (blk < G::NHB) {                          // uniform
#pragma unroll
          for (int cb = 0; cb < CB / 16; ++cb) {
            uint2 hv = project(xhn[i], wvs, bvs, [&](int r) { return 16 * cb + r; });
            if (!((hok >> i) & 1u)) hv = make_uint2(0u, 0u);
            *(uint2*)(Hw + (16 * blk + lq) * CB + 16 * cb + 4 * lg) = hv;
          }
        }
      }
      // Q straight into the operand layout (channels 32hb + 8lg .. +7 of
      // query lq): two products whose D rows are the weight rows 8(i/4) +
      // i%4 and that + 4, so lane lg ends with channels 8lg .. 8lg+3 and
      // 8lg+4 .. 8lg+7 (each element's sum is the same as unpermuted)
      const uint2 q0 = project(xqn, wqs, bqs, [&](int i) { return hb * kHd + 8 * (i >> 2) + (i & 3); });
      const uint2 q1 = project(xqn, wqs, bqs,
                               [&](int i) { return hb * kHd + 8 * (i >> 2) + 4 + (i & 3); });
      qop = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
    }
    __syncthreads();                                 // (XP: every key block is in place)
    if (j + 1 < nu) prefetch(j + 1);
    const uint16_t* Hs = (const uint16_t*)buf;
    const uint16_t* Ks = (const uint16_t*)(buf + G::HALO);
    const uint16_t* Vs = (const uint16_t*)(buf + G::HALO + G::KVB);

    // ---- LePE of this lane's items, in three slices of input rows ----
    float lw[TYW][XG];
#pragma unroll
    for (int r = 0; r < TYW; ++r)
#pragma unroll
      for (int k = 0; k < XG; ++k) lw[r][k] = b0;
    // transposing reads of 4 consecutive halo pixels of one channel: lane i
    // of a 16-lane row addresses pixel xw + i/4 (+4 for the second read),
    // channels (cw & ~15) + 4(i % 4) .. +3, and receives channel cw of the
    // four pixels as two bf16 pairs along x
    const uint16_t* trp = Hs + ((qrow0 + yl) * HW + xw + (lq >> 2)) * CB + (cw & ~15) + 4 * (lane & 3);
    auto conv_rows = [&](int dy0, int dy1) {
#pragma unroll
      for (int dy = 0; dy < TYW + KS - 1; ++dy) {
        if (dy < dy0 || dy >= dy1) continue;
        const uint2 a = lds_read_tr16(trp + (dy * HW) * CB);
        const uint2 b = lds_read_tr16(trp + (dy * HW + 4) * CB);
        const uint32_t p0 = a.x, p1 = a.y, p2 = b.x, p3 = b.y;   // pixel pairs
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const int r = dy - i;
          if (r < 0 || r >= TYW) continue;
          lw[r][0] = dot2(we[i][2], p2, dot2(we[i][1], p1, dot2(we[i][0], p0, lw[r][0])));
          lw[r][1] = dot2(wo[i][2], p2, dot2(wo[i][1], p1, dot2(wo[i][0], p0, lw[r][1])));
          if constexpr (XG == 4) {
            lw[r][2] = dot2(we[i][2], p3, dot2(we[i][1], p2, dot2(we[i][0], p1, lw[r][2])));
            lw[r][3] = dot2(wo[i][2], p3, dot2(wo[i][1], p2, dot2(wo[i][0], p1, lw[r][3])));
          }
        }
      }
    };
    constexpr int NR = TYW + KS - 1;                   // input rows of an item

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
    // K operand of 16-key block kb: lane (lq, lg) holds channels
    // 32hb + 8lg .. +7 of key 16kb + lq
    auto kop = [&](int kb) -> bf16x8 {
      const int key = 16 * kb + lq;
      return *(const bf16x8*)(Ks + key * CB + (((hb * 4 + lg) ^ kswz<GB>(key)) * 8));
    };
    // V^T operands by transposing reads of the row-major V tile: lane (lq, lg)
    // addresses key 4lg + lq/4 (+16 for slots 4-7), channels d0 + 4(lq % 4)
    // .. +3, and receives channel d0 + lq of keys 4lg + 0..3 -- the slot order
    // of P^T (slots e: keys 32h + 4lg + e for e < 4, 32h + 16 + 4lg + e - 4).
    const int vrow = 4 * lg + (lq >> 2);               // key within a 16-key block
    const int vsw = kswz<GB>(vrow);                    // same for vrow + 16m
    const uint16_t* vbase = Vs + vrow * CB + 4 * (lq & 1);
    const int ca = ((hb * 4 + ((lq >> 1) & 1)) ^ vsw) * 8;       // d0 = 32hb
    const int cbo = ((hb * 4 + 2 + ((lq >> 1) & 1)) ^ vsw) * 8;  // d0 = 32hb + 16
    // O^T += V^T P^T and the row sums += ones P^T for keys 32h .. 32h+31
    auto pv_step = [&](int h, const uint32_t* p4) {
      const uint16_t* r0 = vbase + (32 * h) * CB;
      const uint16_t* r1 = r0 + 16 * CB;
      const uint2 a0 = lds_read_tr16(r0 + ca), a1 = lds_read_tr16(r1 + ca);
      const uint2 c0 = lds_read_tr16(r0 + cbo), c1 = lds_read_tr16(r1 + cbo);
      const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
      const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
      const bf16x8 phi = __builtin_bit_cast(bf16x8, make_uint4(p4[0], p4[1], p4[2], p4[3]));
      acc0 = mfma_bf16(va, phi, acc0);                 // O^T rows d = 4lg + e
      acc1 = mfma_bf16(vb, phi, acc1);                 // O^T rows d = 16 + 4lg + e
      accl = mfma_bf16(ones, phi, accl);               // every row: sum over keys
    };
    if constexpr (!G::TWO_PASS) {
      // ---- attention phase 1: S^T = K Q^T, kept in registers ----
      float x[KC / 4];
#pragma unroll
      for (int kb = 0; kb < KC / 16; ++kb) {
        const f32x4 sv = mfma_bf16(kop(kb), qop, f32x4{0.f, 0.f, 0.f, 0.f});
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
#pragma unroll
      for (int h = 0; h < KC / 32; ++h) pv_step(h, ph + 4 * h);
    } else if constexpr (G::ONLINE) {
      // ---- many routed keys, 64 a step: S^T of the step, the running row
      // maximum, the accumulators (O and the row sums alike) rescaled by
      // 2^((m_old - m_new) c) when it grows, numerators against the new
      // maximum (so every weight is at most 1), O^T += V^T P^T ----
      float m = -3.0e38f;
      auto chunk = [&](int ch) {
        float xx[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 sv = mfma_bf16(kop(4 * ch + q), qop, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int e = 0; e < 4; ++e) xx[4 * q + e] = sv[e];
        }
        float mk = xx[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mk = fmaxf(mk, xx[e]);
        mk = fmaxf(mk, xor16(mk));
        mk = fmaxf(mk, xor32(mk));
        const float mn = fmaxf(m, mk);
        if (ch > 0) {
          const float alpha = __builtin_amdgcn_exp2f((m - mn) * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc0[e] *= alpha;
            acc1[e] *= alpha;
            accl[e] *= alpha;
          }
        }
        m = mn;
        const float mc = m * c;
        uint32_t p8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p8[e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(xx[2 * e], c, -mc)),
                              __builtin_amdgcn_exp2f(fmaf(xx[2 * e + 1], c, -mc)));
        pv_step(2 * ch, p8);
        pv_step(2 * ch + 1, p8 + 4);
      };
      static_assert(KC % 64 == 0 && KC / 64 >= 2, "online steps: whole 64-key steps, at least two");
      chunk(0);
      __builtin_amdgcn_sched_barrier(0);
      conv_rows(0, NR / 3);
      __builtin_amdgcn_sched_barrier(0);
      chunk(1);
      __builtin_amdgcn_sched_barrier(0);
      conv_rows(NR / 3, 2 * NR / 3);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ch = 2; ch < KC / 64; ++ch) chunk(ch);
    } else {
      // ---- many routed keys: phase 1 keeps only the row maximum; phase 2
      // computes S^T again, 32 keys a step, into numerators and O ----
      float m = -3.0e38f;
#pragma unroll
      for (int kb = 0; kb < KC / 16; ++kb) {
        const f32x4 sv = mfma_bf16(kop(kb), qop, f32x4{0.f, 0.f, 0.f, 0.f});
        m = fmaxf(m, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      }
      m = fmaxf(m, xor16(m));
      m = fmaxf(m, xor32(m));
      const float mc = m * c;
      __builtin_amdgcn_sched_barrier(0);
      conv_rows(0, NR / 3);
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](int h) {
        const f32x4 s0 = mfma_bf16(kop(2 * h), qop, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 s1 = mfma_bf16(kop(2 * h + 1), qop, f32x4{0.f, 0.f, 0.f, 0.f});
        uint32_t p4[4];
        p4[0] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[0], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(s0[1], c, -mc)));
        p4[1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s0[2], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(s0[3], c, -mc)));
        p4[2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[0], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(s1[1], c, -mc)));
        p4[3] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s1[2], c, -mc)),
                            __builtin_amdgcn_exp2f(fmaf(s1[3], c, -mc)));
        pv_step(h, p4);
      };
#pragma unroll
      for (int h = 0; h < KC / 64; ++h) step(h);
      __builtin_amdgcn_sched_barrier(0);
      conv_rows(NR / 3, 2 * NR / 3);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = KC / 64; h < KC / 32; ++h) step(h);
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(2 * NR / 3, NR);

    // ---- L through the wavefront's tile into the MFMA layout ----
#pragma unroll
    for (int r = 0; r < TYW; ++r)
#pragma unroll
      for (int k = 0; k < XG; ++k) Lw[((yl + r) * WS + xw + k) * LSW + (lane & 31)] = lw[r][k];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    // ---- out = O / l + L, one rounding, 16-byte stores ----
    {
      int b, ry, rx;
      decode(j, b, ry, rx);
      const auto O = image_rsrc(A.out + (size_t)b * img_elems, img_elems * 2);
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
      const uint32_t op = ((ry * HS + q / WS) * A.W + rx * WS + q % WS) * C + cb0 + hb * kHd + ch;
      bstore16<G::OUT_CPOL>(O, q < n ? op * 2 : kOob, ov);
    }
    if constexpr (!G::DB) __syncthreads();         // the buffer is restaged next
  }
}

template <class G>
hipError_t region_launch_images(RegionArgs a, int cus_per_xcd, int min_bpx, hipStream_t st) {
  a.per_xcd = (int)units_per_xcd(a.units, kXcds, G::NCB);
  // LDS with the routing table sized for the fewest workgroups an XCD gets
  // (one per CU, rounded to whole channel blocks): an upper bound
  const int maxu_bound = (int)units_per_workgroup(a.per_xcd, min_bpx);
  size_t lds = G::IT_OFF + (size_t)maxu_bound * G::TOPK * sizeof(int);
  const void* fn = reinterpret_cast<const void*>(&attend_region_kernel<G>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_region_kernel<G>, kThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  int bpx = cus_per_xcd * per_cu;
  bpx = bpx / G::NCB * G::NCB;
  if (bpx < G::NCB) bpx = G::NCB;
  if (bpx > a.per_xcd) bpx = a.per_xcd;
  a.bpx = bpx;
  const int maxu = (int)units_per_workgroup(a.per_xcd, bpx);
  lds = G::IT_OFF + (size_t)maxu * G::TOPK * sizeof(int);
  hipLaunchKernelGGL(attend_region_kernel<G>, dim3((unsigned)(bpx * kXcds)), dim3(kThreads), lds,
                     st, a);
  return hipGetLastError();
}

// A batch runs as launches over image ranges small enough that a
// workgroup's routing table stays within kTableBytes (one launch for every
// batch of the workload shapes).
template <class G>
hipError_t region_launch(RegionArgs a, int B, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int cus_per_xcd = cus / kXcds > 0 ? cus / kXcds : 1;
  const int min_bpx = cus_per_xcd / G::NCB * G::NCB > G::NCB ? cus_per_xcd / G::NCB * G::NCB
                                                              : G::NCB;
  const long long upi = (long long)a.R * G::NCB;
  const int per = images_per_launch(B, upi, kXcds, G::NCB, min_bpx, G::TOPK, kTableBytes);
  if (per < 1) return hipErrorNotSupported;
  const size_t img_elems = (size_t)a.H * a.W * G::C;
  for (int b0 = 0; b0 < B; b0 += per) {
    const int nb = B - b0 < per ? B - b0 : per;
    RegionArgs c = a;
    c.q += b0 * img_elems; c.k += b0 * img_elems; c.v += b0 * img_elems;
    c.out += b0 * img_elems;
    c.idx += (size_t)b0 * a.R * G::TOPK;
    c.units = (int)(nb * upi);
    e = region_launch_images<G>(c, cus_per_xcd, min_bpx, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The shapes with a dedicated kernel (d = 32, 5x5 LePE): the BiFormer stage
// shapes at 224^2 (56^2 / 28^2 / 14^2 maps, S = 7, top-k 1 / 4 / 16) and the
// 512^2 segmentation shape (128^2 map, S = 16, top-k 4).  Four tasks per
// unit: one head for the 8x8 regions, four heads for the 4x4 and 2x2 ones.
#ifndef BRA_DB_ST1
#define BRA_DB_ST1 false
#endif
#ifndef BRA_DB_DENSE
#define BRA_DB_DENSE false
#endif
using St1 = Rc<64, 32, 8, 8, 1, 5, BRA_DB_ST1, 4>;
using St2 = Rc<128, 128, 4, 4, 4, 5, false>;
using St3 = Rc<256, 128, 2, 2, 16, 5, false>;
using Dense = Rc<64, 32, 8, 8, 4, 5, BRA_DB_DENSE, 3, true>;
// the rest of the 8x8-region family (C = 32..128 in heads of 32, top-1, 2
// or 4): units of one head, so only the image stride changes with C; top-1
// as St1 (four workgroups a CU), top-2 (128 keys, S^T held) and top-4 (the
// one-pass softmax) at three, top-4 with the dense shape's non-temporal
// stores
template <int C, int TOPK>
using Rc8 = Rc<C, 32, 8, 8, TOPK, 5, false, TOPK == 1 ? 4 : 3, TOPK == 4>;
// the module's fused form of St1: Q and K projected from x in the kernel
using StX1 = Rc<64, 32, 8, 8, 1, 5, false, 3, false, true>;

}  // namespace

hipError_t launch_attend_region(const void* q, const void* k, const void* v, const int32_t* idx,
                                const Shape& s, float attn_scale, const float* w,
                                const float* bias, int ks, void* out, hipStream_t st) {
  if (!w || s.C != s.heads * kHd) return hipErrorNotSupported;
  // buffer offsets of one image (bytes) stay below the out-of-range marker
  if ((long long)s.H * s.W * s.C * 2 >= (long long)kOob) return hipErrorNotSupported;
  RegionArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.idx = idx; a.out = (uint16_t*)out; a.w = w; a.bias = bias;
  a.wq = a.wk = a.wv = nullptr;
  a.bq = a.bk = a.bv = nullptr;
  a.H = s.H; a.W = s.W; a.S = s.S; a.R = s.R; a.Hf = s.Hf;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.f_R = make_fastdiv(s.R);
  a.f_S = make_fastdiv(s.S);
  if (s.Hf < 1 || s.Hf % s.hs || s.H % s.Hf) return hipErrorInvalidValue;
  a.f_syf = make_fastdiv(s.Hf / s.hs);
  a.per_xcd = a.bpx = 0;
  auto is = [&](int C, int hs, int ws, int topk, int kks) {
    return s.C == C && s.hs == hs && s.ws == ws && s.topk == topk && ks == kks;
  };
  if (is(St1::C, St1::HS, St1::WS, St1::TOPK, St1::KS)) {
    return region_launch<St1>(a, s.B, st);
  }
  if (is(St2::C, St2::HS, St2::WS, St2::TOPK, St2::KS)) {
    return region_launch<St2>(a, s.B, st);
  }
  if (is(St3::C, St3::HS, St3::WS, St3::TOPK, St3::KS)) {
    return region_launch<St3>(a, s.B, st);
  }
  if (is(Dense::C, Dense::HS, Dense::WS, Dense::TOPK, Dense::KS)) {
    return region_launch<Dense>(a, s.B, st);
  }
  if (s.hs == 8 && s.ws == 8 && ks == 5) {
#define BRA_RC8(CC)                                                  \
    if (s.C == CC) {                                                 \
      if (s.topk == 1) return region_launch<Rc8<CC, 1>>(a, s.B, st); \
      if (s.topk == 2) return region_launch<Rc8<CC, 2>>(a, s.B, st); \
      if (s.topk == 4) return region_launch<Rc8<CC, 4>>(a, s.B, st); \
    }
    BRA_RC8(32) BRA_RC8(64) BRA_RC8(96) BRA_RC8(128) BRA_RC8(192) BRA_RC8(256)
#undef BRA_RC8
  }
  return hipErrorNotSupported;
}

bool attend_xproj_ok(const Shape& s, const float* w, int ks) {
  return w && s.C == StX1::C && s.C == s.heads * kHd && s.hs == StX1::HS && s.ws == StX1::WS &&
         s.topk == StX1::TOPK && ks == StX1::KS && s.Hf == s.H &&
         (long long)s.H * s.W * s.C * 2 < (long long)kOob;
}

hipError_t launch_attend_xproj(const void* x, const void* w_qkv, const float* b_qkv,
                               const int32_t* idx, const Shape& s, float attn_scale,
                               const float* w, const float* bias, int ks, void* out,
                               hipStream_t st) {
  if (!attend_xproj_ok(s, w, ks)) return hipErrorNotSupported;
  RegionArgs a;
  a.q = a.k = a.v = (const uint16_t*)x;
  a.idx = idx; a.out = (uint16_t*)out; a.w = w; a.bias = bias;
  a.wq = (const uint16_t*)w_qkv;
  a.wk = (const uint16_t*)w_qkv + (size_t)s.C * s.C;
  a.wv = (const uint16_t*)w_qkv + (size_t)2 * s.C * s.C;
  a.bq = b_qkv;
  a.bk = b_qkv ? b_qkv + s.C : nullptr;
  a.bv = b_qkv ? b_qkv + 2 * s.C : nullptr;
  a.H = s.H; a.W = s.W; a.S = s.S; a.R = s.R; a.Hf = s.Hf;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.f_R = make_fastdiv(s.R);
  a.f_S = make_fastdiv(s.S);
  a.f_syf = make_fastdiv(s.Hf / s.hs);
  a.per_xcd = a.bpx = 0;
  return region_launch<StX1>(a, s.B, st);
}

}  // namespace bra
