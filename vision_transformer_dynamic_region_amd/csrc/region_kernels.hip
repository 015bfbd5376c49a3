// Fused gather-attention + LePE for bf16 inputs whose region shape is known at
// compile time (the BiFormer stage shapes): one persistent, software-pipelined
// kernel per shape.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3: gather of the routed regions' tokens, softmax attention, LePE added to
// the output), p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉
// Transformer的计算范式" (§4: the depthwise LePE conv on V), p5 = hyper.ai
// abstract of BiFormer (token-to-token attention over the union of the routed
// regions).
//
// What a workgroup does.  A unit is (image, query region, block of CB
// channels = CB/32 heads).  The units of an XCD are dealt round-robin to that
// XCD's workgroups, so at any moment one XCD works on neighbouring regions of
// one image and its L2 serves their shared halo rows and routed regions.  Per
// unit:
//   1. the unit's V halo (the region plus KS/2 pixels each side, zero
//      outside the image) goes from registers to LDS as float32, the routed
//      regions' K rows to LDS row-major (16-byte chunks XOR-swizzled by row),
//      their V rows to LDS transposed [channel][key]; barrier;
//   2. the global loads of the next unit (its query operands, routed K/V
//      vectors and halo) are issued into registers;
//   3. attention: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (one query per
//      lane column), softmax in float32 with the scale folded into exp2,
//      O^T = V^T P^T with P rounded to bf16;
//   4. LePE: each thread convolves one channel pair over one column of TY
//      rows from the float32 halo, with its 2 x KS x KS weights held in
//      registers for the life of the workgroup; the float32 L tile goes to
//      LDS; barrier;
//   5. out = O / l + L, rounded once to bf16, stored.
// Nothing but the output is written to memory: the gathered K/V exist only
// in LDS.

#include "device_common.h"

namespace bra {
namespace {

constexpr int kHd = 32;    // head width

// Rows per LePE item: the smallest divisor TY of HS such that the items
// (channel pairs x columns x row blocks) fit one per thread.
constexpr int pick_ty(int cw, int hs) {
  for (int ty = 1; ty <= hs; ++ty)
    if (hs % ty == 0 && cw * (hs / ty) <= kThreads) return ty;
  return hs;
}

// OCC: workgroups per CU the layout is sized for.  With OCC >= 3 the L tile
// reuses the K/V area (one more barrier per unit) and registers are capped
// accordingly.
#ifndef BRA_LEPE_BF16W
#define BRA_LEPE_BF16W 1
#endif

// W16: LePE on v_dot2_f32_bf16 (weights rounded once to bf16, products exact,
// float32 accumulation) from a bf16 halo; otherwise float32 FMAs from a
// float32 halo.
template <int C_, int CB_, int HS_, int WS_, int TOPK_, int KS_, int OCC_ = 2,
          bool W16_ = BRA_LEPE_BF16W>
struct Rc {
  static constexpr int C = C_, CB = CB_, HS = HS_, WS = WS_, TOPK = TOPK_, KS = KS_;
  static constexpr int OCC = OCC_;
  static constexpr bool W16 = W16_;
  static constexpr bool L_ALIAS = OCC_ >= 3;
  static constexpr int NCB = C / CB;               // channel blocks per region
  static constexpr int n = HS * WS;                // queries per region
  static constexpr int KC = TOPK * n;              // routed keys, all in LDS at once
  static constexpr int NQB = (n + 15) / 16;        // 16-query blocks
  static constexpr int HB = CB / kHd;              // heads per unit
  static constexpr int TASKS = NQB * HB;
  static constexpr int TPW = (TASKS + kWaves - 1) / kWaves;
  static constexpr int P = KS / 2;
  static constexpr int KK = KS * KS;
  static constexpr int HH = HS + KS - 1, HW = WS + KS - 1;
  static constexpr int GB = CB / 8;                // 16-byte vectors per pixel
  static constexpr int PSTEP = kThreads / GB;      // pixels per staging pass
  static constexpr int HPT = (HH * HW + PSTEP - 1) / PSTEP;
  static constexpr int KPT = (KC + PSTEP - 1) / PSTEP;
  static constexpr int CP = CB / 2;                // LePE channel pairs
  static constexpr int TY = pick_ty(CP * WS, HS);
  static constexpr int ITEMS = CP * WS * (HS / TY);
  static constexpr int LS = CB + 4;                // L row stride (floats)
  // dot2 LePE items: one channel, XG columns (tap pairs along x), TYW rows
  static constexpr int XG = WS % 4 == 0 ? 4 : WS;
  static constexpr int NXG = WS / XG;
  static constexpr int TYW = pick_ty(CB * NXG, HS);
  static constexpr int ITEMS_W = CB * NXG * (HS / TYW);
  static constexpr int HALO_BYTES = HH * HW * CB * (W16 ? 2 : 4);
  static constexpr int K_OFF = HALO_BYTES > KK * CB * 4 ? HALO_BYTES : KK * CB * 4;
  static constexpr int V_OFF = K_OFF + KC * CB * 2;
  static constexpr int KV_END = V_OFF + KC * CB * 2;
  static constexpr int L_OFF = L_ALIAS ? K_OFF : KV_END;
  static constexpr int IT_OFF = L_ALIAS ? (KV_END > L_OFF + n * LS * 4 ? KV_END : L_OFF + n * LS * 4)
                                        : L_OFF + n * LS * 4;

  static_assert(C % CB == 0 && CB % kHd == 0, "channel blocking");
  static_assert(kThreads % GB == 0, "a thread stages one fixed 16-byte vector of a pixel");
  static_assert(KC % 32 == 0 && KC <= 256, "routed keys: a multiple of 32, one softmax step");
  static_assert(W16 || (kThreads % CP == 0 && ITEMS <= kThreads), "one LePE item per thread");
  static_assert(!W16 || (KS == 5 && CB % 16 == 0 && (XG == 4 || XG == 2) && ITEMS_W <= kThreads &&
                         kThreads % CB == 0),
                "dot2 LePE: 5x5 taps, 16-channel lane rows, one item per thread");
};

// K tile swizzle: chunk g (16 bytes) of key row kk sits at chunk g ^ kswz(kk),
// so the 16 rows one operand load reads fall into 16 distinct bank groups.
template <int GB>
__device__ __forceinline__ int kswz(int kk) {
  if constexpr (GB >= 16) return kk & 15;
  else if constexpr (GB == 8) return (kk >> 1) & 7;
  else return (kk >> 2) & 3;
}

// Float32 halo pixel layout: the 16-byte vector g of a pixel (channels
// 8g..8g+7) is split so that channels 8g..8g+3 sit at floats 4g..4g+3 and
// 8g+4..8g+7 at CB/2 + 4g..: the two 16-byte LDS writes of consecutive lanes
// are then contiguous.  hpos gives a channel's float position.
template <int CB>
__device__ __forceinline__ int hpos(int c) {
  return ((c & 4) ? CB / 2 : 0) + (c >> 3) * 4 + (c & 3);
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
  int H, W, S, R;
  float scale_log2;     // attn_scale * log2(e)
  int units;            // B * R * NCB
  int per_xcd;          // units per XCD (a multiple of NCB)
  int bpx;              // workgroups per XCD (a multiple of NCB)
  FastDiv f_R, f_S;
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
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}

template <class G>
__global__ __launch_bounds__(kThreads, G::OCC) void attend_region_kernel(RegionArgs A) {
  constexpr int C = G::C, CB = G::CB, HS = G::HS, WS = G::WS, TOPK = G::TOPK;
  constexpr int n = G::n, KC = G::KC, NQB = G::NQB, TASKS = G::TASKS, TPW = G::TPW;
  constexpr int P = G::P, KS = G::KS, KK = G::KK, HH = G::HH, HW = G::HW, GB = G::GB;
  constexpr int PSTEP = G::PSTEP, HPT = G::HPT, KPT = G::KPT, CP = G::CP, TY = G::TY;
  constexpr int LS = G::LS, NCB = G::NCB;
  extern __shared__ __align__(16) unsigned char lds[];
  float* Hs = (float*)lds;
  uint16_t* Ks = (uint16_t*)(lds + G::K_OFF);
  uint16_t* Vs = (uint16_t*)(lds + G::V_OFF);
  float* Ls = (float*)(lds + G::L_OFF);
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
  // this block's LePE weights, transposed to [tap][channel] in the halo area
  // (consecutive threads write consecutive LDS words)
  for (int e = tid; e < KK * CB; e += kThreads) {
    const int t = e / CB, c = e - t * CB;
    Hs[e] = A.w[(size_t)(cb0 + c) * KK + t];
  }
  __syncthreads();

  // LePE item of this thread.
  //  float32 path: channel pair cp, column xc, rows y0 .. y0+TY-1;
  //  dot2 path: channel cw, columns xw .. xw+XG-1, rows yw .. yw+TYW-1.
  constexpr int XG = G::XG, NXG = G::NXG, TYW = G::TYW;
  const bool conv_on = G::W16 ? (G::ITEMS_W == kThreads || tid < G::ITEMS_W)
                              : (G::ITEMS == kThreads || tid < G::ITEMS);
  const int cp = tid % CP, xc = (tid / CP) % WS, y0 = (tid / (CP * WS)) * TY;
  const int cw = tid % CB, xw = ((tid / CB) % NXG) * XG, yw = (tid / (CB * NXG)) * TYW;
  float wr[G::W16 ? 1 : KK][2];
  // dot2 weights per kernel row i: for an even output column the tap pairs
  // (w0,w1) (w2,w3) (w4,0) over input pairs (x,x+1) (x+2,x+3) (x+4,x+5); for
  // the odd column after it (0,w0) (w1,w2) (w3,w4) over the same pairs
  uint32_t we[G::W16 ? KS : 1][3], wo[G::W16 ? KS : 1][3];
  float b0 = 0.f, b1 = 0.f;
  if constexpr (G::W16) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      float t[5];
#pragma unroll
      for (int jx = 0; jx < 5; ++jx) t[jx] = Hs[(i * KS + jx) * CB + cw];
      we[i][0] = pack_bf16x2(t[0], t[1]);
      we[i][1] = pack_bf16x2(t[2], t[3]);
      we[i][2] = pack_bf16x2(t[4], 0.f);
      wo[i][0] = pack_bf16x2(0.f, t[0]);
      wo[i][1] = pack_bf16x2(t[1], t[2]);
      wo[i][2] = pack_bf16x2(t[3], t[4]);
    }
    if (A.bias) b0 = A.bias[cb0 + cw];
  } else {
#pragma unroll
    for (int t = 0; t < KK; ++t) {
      const float2 u = *(const float2*)(Hs + t * CB + 2 * cp);
      wr[t][0] = u.x;
      wr[t][1] = u.y;
    }
    if (A.bias) {
      b0 = A.bias[cb0 + 2 * cp];
      b1 = A.bias[cb0 + 2 * cp + 1];
    }
  }

  const int g = tid % GB, pk = tid / GB;           // staged vector: pixel pk + PSTEP*i, chunk g
  auto decode = [&](int j, int& b, int& ry, int& rx) {
    const int br = (u0 + j * A.bpx) / NCB;
    b = fdiv(br, A.f_R);
    const int r = br - b * A.R;
    ry = fdiv(r, A.f_S);
    rx = r - ry * A.S;
  };

  const uint32_t img_elems = (uint32_t)A.H * A.W * C;
  uint4 qn[TPW], kn[KPT], vn[KPT], hn[G::HPT];
  auto prefetch = [&](int j) {
    int b, ry, rx;
    decode(j, b, ry, rx);
    const size_t img = (size_t)b * img_elems;
    const auto Q = image_rsrc(A.q + img, img_elems * 2);
    const auto K = image_rsrc(A.k + img, img_elems * 2);
    const auto V = image_rsrc(A.v + img, img_elems * 2);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + kWaves * i;
      const int qb = t % NQB, hb = t / NQB, q = qb * 16 + lq;
      const bool ok = (TASKS % kWaves == 0 || t < TASKS) && q < n;
      const uint32_t off = ((ry * HS + q / WS) * A.W + rx * WS + q % WS) * C + cb0 + hb * kHd + 8 * lg;
      qn[i] = bload16(Q, ok ? off * 2 : kOob);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int kk = pk + PSTEP * i;
      const int tj = kk / n, tok = kk % n;
      const uint32_t off =
          (PSTEP * (i + 1) <= KC || kk < KC) ? (itab[j * TOPK + tj] + ((tok / WS) * A.W + tok % WS) * C + cb0 + g * 8) * 2 : kOob;
      kn[i] = bload16(K, off);
      vn[i] = bload16(V, off);
    }
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int pix = pk + PSTEP * i;
      const int hy = pix / HW, hx = pix % HW;
      const int y = ry * HS - P + hy, x = rx * WS - P + hx;
      // one unsigned compare per bound; & rather than && keeps this branch-free
      const bool ok = (PSTEP * (i + 1) <= HH * HW || pix < HH * HW) & ((unsigned)y < (unsigned)A.H) &
                      ((unsigned)x < (unsigned)A.W);
      hn[i] = bload16(V, ok ? (uint32_t)((__umul24(y, A.W) + x) * C + cb0 + g * 8) * 2 : kOob);
    }
  };

  bf16x8 qop[TPW];
  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int pix = pk + PSTEP * i;                 // pk < PSTEP
      if (PSTEP * (i + 1) <= HH * HW || pix < HH * HW) {
        const uint4 u = hn[i];
        if constexpr (G::W16) {
          *(uint4*)((uint16_t*)Hs + pix * CB + g * 8) = u;
        } else {
          float* d = Hs + pix * CB + g * 4;
          *(float4*)d = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
          *(float4*)(d + CB / 2) = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
        }
      }
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
#pragma unroll
    for (int i = 0; i < TPW; ++i) qop[i] = __builtin_bit_cast(bf16x8, qn[i]);
  };

  const float c = A.scale_log2;
  prefetch(0);
  __syncthreads();                                  // weights read; the halo area is free

  for (int j = 0; j < nu; ++j) {
    commit();
    __syncthreads();
    if (j + 1 < nu) prefetch(j + 1);

    // ---- attention over the KC routed keys (one softmax step) and the
    // LePE convolution, interleaved phase by phase: the convolution's
    // independent FMAs fill the latency of the MFMA -> softmax -> MFMA chain.
    // sched_barrier keeps the compiler from regrouping the phases.
    f32x4 acc0[TPW], acc1[TPW];
    float lsum[TPW];
    float x[TPW][KC / 4];
    uint32_t ph[TPW][KC / 8];                         // bf16 pairs of P, slot order

    float la[TY][2];
    float lw[TYW][XG];
#pragma unroll
    for (int r = 0; r < TY; ++r) {
      la[r][0] = b0;
      la[r][1] = b1;
    }
#pragma unroll
    for (int r = 0; r < TYW; ++r)
#pragma unroll
      for (int k = 0; k < XG; ++k) lw[r][k] = b0;
    const float* hp = Hs + (y0 * HW + xc) * CB + hpos<CB>(2 * cp);
    // dot2 path: transposing reads of 4 consecutive halo pixels of one
    // channel.  Lane i of a 16-lane row addresses pixel xw + i/4 (+4 for the
    // second read), channels (cw & ~15) + 4(i % 4) .. +3, and receives
    // channel cw of the four pixels: two bf16 pairs along x.
    const uint16_t* trp = (const uint16_t*)Hs + (yw * HW + xw + ((tid & 15) >> 2)) * CB +
                          (cw & ~15) + 4 * (tid & 3);
    // LePE input rows dy0 .. dy1-1 of this thread's item
    auto conv_rows = [&](int dy0, int dy1) {
      if (!conv_on) return;
      if constexpr (G::W16) {
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
        return;
      }
#pragma unroll
      for (int dy = 0; dy < TY + KS - 1; ++dy) {
        if (dy < dy0 || dy >= dy1) continue;
        float2 vv[KS];
#pragma unroll
        for (int jx = 0; jx < KS; ++jx) vv[jx] = *(const float2*)(hp + (dy * HW + jx) * CB);
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          const int r = dy - i;
          if (r < 0 || r >= TY) continue;
#pragma unroll
          for (int jx = 0; jx < KS; ++jx) {
            la[r][0] = fmaf(wr[i * KS + jx][0], vv[jx].x, la[r][0]);
            la[r][1] = fmaf(wr[i * KS + jx][1], vv[jx].y, la[r][1]);
          }
        }
      }
    };
    constexpr int NR = (G::W16 ? TYW : TY) + KS - 1;   // input rows of an item

    // phase 1: S^T = K Q^T for every task
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[i] = 0.f;
      const int t = wave + kWaves * i;
      if (TASKS % kWaves != 0 && t >= TASKS) continue;   // uniform over the wave
      const int hb = t / NQB;
#pragma unroll
      for (int kb = 0; kb < KC / 16; ++kb) {
        const int key = 16 * kb + lq;
        const bf16x8 ka =
            *(const bf16x8*)(Ks + key * CB + (((hb * 4 + lg) ^ kswz<GB>(key)) * 8));
        const f32x4 sv = mfma_bf16(ka, qop[i], f32x4{0.f, 0.f, 0.f, 0.f});
        // lane holds keys 16*kb + 4*lg + e of query lq
#pragma unroll
        for (int e = 0; e < 4; ++e) x[i][4 * kb + e] = sv[e];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(0, NR / 3);
    __builtin_amdgcn_sched_barrier(0);

    // phase 2: softmax numerators, rounded to bf16 in P^T slot order
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + kWaves * i;
      if (TASKS % kWaves != 0 && t >= TASKS) continue;
      float m = x[i][0];
#pragma unroll
      for (int e = 1; e < KC / 4; ++e) m = fmaxf(m, x[i][e]);
      m = fmaxf(m, xor16(m));
      m = fmaxf(m, xor32(m));
      const float mc = m * c;
      float p[KC / 4];
#pragma unroll
      for (int e = 0; e < KC / 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[i][e], c, -mc));
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < KC / 4; ++e) ps += p[e];
      lsum[i] = ps;
#pragma unroll
      for (int e = 0; e < KC / 8; ++e) ph[i][e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(NR / 3, 2 * NR / 3);
    __builtin_amdgcn_sched_barrier(0);

    // phase 3: O^T += V^T P^T.  V^T operands come straight from the
    // row-major V tile by transposing reads: lane (lq, lg) addresses key
    // 4lg + lq/4 (+16 for slots 4-7), channels d0 + 4(lq % 4) .. +3, and
    // receives channel d0 + lq of keys 4lg + 0..3 -- the slot order of P^T
    // (slots e: keys 32h + 4lg + e for e < 4, 32h + 16 + 4lg + e - 4 after).
    const int vrow = 4 * lg + (lq >> 2);                   // key within a 16-key block
    const int vsw = kswz<GB>(vrow);                        // same for vrow + 16m
    const uint16_t* vbase = Vs + vrow * CB + 4 * (lq & 1);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + kWaves * i;
      if (TASKS % kWaves != 0 && t >= TASKS) continue;
      const int hb = t / NQB;
      const int ca = ((hb * 4 + ((lq >> 1) & 1)) ^ vsw) * 8;       // d0 = 32hb
      const int cb = ((hb * 4 + 2 + ((lq >> 1) & 1)) ^ vsw) * 8;   // d0 = 32hb + 16
#pragma unroll
      for (int h = 0; h < KC / 32; ++h) {
        const uint16_t* r0 = vbase + (32 * h) * CB;
        const uint16_t* r1 = r0 + 16 * CB;
        const uint2 a0 = lds_read_tr16(r0 + ca), a1 = lds_read_tr16(r1 + ca);
        const uint2 c0 = lds_read_tr16(r0 + cb), c1 = lds_read_tr16(r1 + cb);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
        const bf16x8 phi = __builtin_bit_cast(
            bf16x8, make_uint4(ph[i][4 * h], ph[i][4 * h + 1], ph[i][4 * h + 2], ph[i][4 * h + 3]));
        acc0[i] = mfma_bf16(va, phi, acc0[i]);      // O^T rows d = 4lg + e
        acc1[i] = mfma_bf16(vb, phi, acc1[i]);      // O^T rows d = 16 + 4lg + e
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    conv_rows(2 * NR / 3, NR);

    // The L tile has its own area unless it reuses K/V (then every wave must
    // be done with the attention first).  Either way the epilogue of the
    // previous unit ended before this unit's first barrier.
    if constexpr (G::L_ALIAS) __syncthreads();
    if (conv_on) {
      if constexpr (G::W16) {
#pragma unroll
        for (int r = 0; r < TYW; ++r)
#pragma unroll
          for (int k = 0; k < XG; ++k) Ls[((yw + r) * WS + xw + k) * LS + cw] = lw[r][k];
      } else {
#pragma unroll
        for (int r = 0; r < TY; ++r)
          *(float2*)(Ls + ((y0 + r) * WS + xc) * LS + 2 * cp) = make_float2(la[r][0], la[r][1]);
      }
    }
    __syncthreads();   // L complete; halo and K/V free for the next unit

    // ---- out = O / l + L, one rounding ----
    int b, ry, rx;
    decode(j, b, ry, rx);
    const auto O = image_rsrc(A.out + (size_t)b * img_elems, img_elems * 2);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + kWaves * i;
      if (TASKS % kWaves != 0 && t >= TASKS) continue;
      const int qb = t % NQB, hb = t / NQB, q = qb * 16 + lq;
      float l = lsum[i];
      l += xor16(l);
      l += xor32(l);
      const float inv = __builtin_amdgcn_rcpf(l);
      const float* lp = Ls + (q < n ? q : 0) * LS + hb * kHd;   // rows >= n: not stored
      const float4 a0 = *(const float4*)(lp + 4 * lg);
      const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
      uint32_t o0x = pack_bf16x2(fmaf(acc0[i][0], inv, a0.x), fmaf(acc0[i][1], inv, a0.y));
      uint32_t o0y = pack_bf16x2(fmaf(acc0[i][2], inv, a0.z), fmaf(acc0[i][3], inv, a0.w));
      uint32_t o1x = pack_bf16x2(fmaf(acc1[i][0], inv, a1.x), fmaf(acc1[i][1], inv, a1.y));
      uint32_t o1y = pack_bf16x2(fmaf(acc1[i][2], inv, a1.z), fmaf(acc1[i][3], inv, a1.w));
      // Lane rows lg, lg^1 trade halves: even rows end up with channels
      // 4lg..4lg+7, odd rows with 16+4(lg-1)..16+4lg+3 -- 16 contiguous bytes.
      const auto sx = __builtin_amdgcn_permlane16_swap(o0x, o1x, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(o0y, o1y, false, false);
      const bool odd = lg & 1;
      const uint4 ov = odd ? make_uint4(sx[0], sy[0], o1x, o1y) : make_uint4(o0x, o0y, sx[1], sy[1]);
      const int ch = odd ? 16 + 4 * (lg - 1) : 4 * lg;
      const uint32_t op = ((ry * HS + q / WS) * A.W + rx * WS + q % WS) * C + cb0 + hb * kHd + ch;
      bstore16(O, q < n ? op * 2 : kOob, ov);
    }
    if constexpr (G::L_ALIAS) __syncthreads();   // L read before K/V are restaged
  }
}

template <class G>
hipError_t region_launch(RegionArgs a, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int cus_per_xcd = cus / kXcds > 0 ? cus / kXcds : 1;
  a.per_xcd = (a.units + kXcds - 1) / kXcds;
  a.per_xcd = (a.per_xcd + G::NCB - 1) / G::NCB * G::NCB;
  // LDS with the routing table sized for one workgroup per CU (an upper bound)
  const int maxu_bound = (a.per_xcd + cus_per_xcd - 1) / cus_per_xcd;
  size_t lds = G::IT_OFF + (size_t)maxu_bound * G::TOPK * sizeof(int);
  const void* fn = reinterpret_cast<const void*>(&attend_region_kernel<G>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
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
  const int maxu = (a.per_xcd + bpx - 1) / bpx;
  lds = G::IT_OFF + (size_t)maxu * G::TOPK * sizeof(int);
  hipLaunchKernelGGL(attend_region_kernel<G>, dim3((unsigned)(bpx * kXcds)), dim3(kThreads), lds,
                     st, a);
  return hipGetLastError();
}

// The shapes with a dedicated kernel: the BiFormer stage shapes at 224^2
// (56^2 / 28^2 / 14^2 maps, S = 7, top-k 1 / 4 / 16, d = 32) with 5x5 LePE.
#ifndef BRA_OCC_ST1
#define BRA_OCC_ST1 2
#endif
#ifndef BRA_CB_ST1
#define BRA_CB_ST1 64
#endif
#ifndef BRA_CB_ST2
#define BRA_CB_ST2 128
#endif
#ifndef BRA_OCC_ST2
#define BRA_OCC_ST2 2
#endif
#ifndef BRA_OCC_ST3
#define BRA_OCC_ST3 2
#endif
using St1 = Rc<64, BRA_CB_ST1, 8, 8, 1, 5, BRA_OCC_ST1>;
using St2 = Rc<128, BRA_CB_ST2, 4, 4, 4, 5, BRA_OCC_ST2>;
using St3 = Rc<256, 128, 2, 2, 16, 5, BRA_OCC_ST3>;
// the 512^2 segmentation shape: 128^2 map, S = 16, top-k 4 (256 keys), d = 32
using Dense = Rc<64, 32, 8, 8, 4, 5>;

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
  a.H = s.H; a.W = s.W; a.S = s.S; a.R = s.R;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.f_R = make_fastdiv(s.R);
  a.f_S = make_fastdiv(s.S);
  a.per_xcd = a.bpx = 0;
  auto is = [&](int C, int hs, int ws, int topk, int kks) {
    return s.C == C && s.hs == hs && s.ws == ws && s.topk == topk && ks == kks;
  };
  if (is(St1::C, St1::HS, St1::WS, St1::TOPK, St1::KS)) {
    a.units = s.B * s.R * St1::NCB;
    return region_launch<St1>(a, st);
  }
  if (is(St2::C, St2::HS, St2::WS, St2::TOPK, St2::KS)) {
    a.units = s.B * s.R * St2::NCB;
    return region_launch<St2>(a, st);
  }
  if (is(St3::C, St3::HS, St3::WS, St3::TOPK, St3::KS)) {
    a.units = s.B * s.R * St3::NCB;
    return region_launch<St3>(a, st);
  }
  if (is(Dense::C, Dense::HS, Dense::WS, Dense::TOPK, Dense::KS)) {
    a.units = s.B * s.R * Dense::NCB;
    return region_launch<Dense>(a, st);
  }
  return hipErrorNotSupported;
}

}  // namespace bra
