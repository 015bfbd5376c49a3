// Gather-attention and LePE kernels of the BRA forward pass (gfx950).
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析",
// p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的
// 计算范式", p5 = hyper.ai abstract of arXiv 2303.08810.

#include "device_common.h"
#include "launch_plan.h"

namespace bra {
namespace {

// ---------------------------------------------------------------------------
// LePE arithmetic shared by the fused attention epilogue and the standalone
// kernel (p2 §4 depthwise Conv2d with zero padding ks//2 and one filter per
// channel; p1 §3 adds it to the attention output):
//   L[y,x,c] = bias[c] + sum_{i,j} w[c,i,j] * V[y+i-ks/2, x+j-ks/2, c]
// Both stage a zero-padded tile of V (th + ks - 1 rows by tw + ks - 1
// columns) and the weights in LDS, cut into slices of 32 channels:
//   tile    [slice][row][col][32]   (elements)
//   weights [slice][tap][32]        (floats)
// so that every offset inside a slice row is a compile-time constant.  A
// thread owns 2 channels of one column over TY output rows and walks the
// TY + ks - 1 input rows once: every input row feeds each output row it
// touches, so a V element is read ks times per strip, not ks*ks times.  Its
// 2*ks*ks weights stay in registers.  Lanes run over the 16 channel pairs of
// a slice, then columns, so a wavefront reads 4 whole pixel slices.  th must
// be a multiple of TY.
// ---------------------------------------------------------------------------
constexpr int kSlice = 32;

template <bool BF16, int KS, int TY, typename Emit>
__device__ __forceinline__ void conv_tile(const void* Hs, const float* Wt, const float* bias,
                                          int c_base, int th, int tw, int nslices,
                                          const FastDiv& f_tw, const FastDiv& f_ns, Emit emit) {
  using T = typename Elem<BF16>::T;
  const int hw = tw + KS - 1, hh = th + KS - 1;
  const int items = 16 * tw * nslices * (th / TY);
  const int rstride = hw * kSlice;               // elements per staged row
  for (int item = threadIdx.x; item < items; item += kThreads) {
    const int cp = item & 15, rest = item >> 4;
    const int rest2 = fdiv(rest, f_tw);
    const int x = rest - rest2 * tw;
    const int sidx = fdiv(rest2, f_ns);
    const int slice = rest2 - sidx * nslices;
    const int y0 = sidx * TY;
    const int cl = 2 * cp;                       // channel pair inside the slice
    float wr[KS * KS][2];
    const float* wp = Wt + slice * (KS * KS * kSlice) + cl;
#pragma unroll
    for (int tap = 0; tap < KS * KS; ++tap) {
      const float2 u = *(const float2*)(wp + tap * kSlice);
      wr[tap][0] = u.x;
      wr[tap][1] = u.y;
    }
    float acc[TY][2];
    float b0 = 0.f, b1 = 0.f;
    if (bias) {
      b0 = bias[c_base + slice * kSlice + cl];
      b1 = bias[c_base + slice * kSlice + cl + 1];
    }
#pragma unroll
    for (int r = 0; r < TY; ++r) {
      acc[r][0] = b0;
      acc[r][1] = b1;
    }
    const T* p = (const T*)Hs + ((slice * hh + y0) * hw + x) * kSlice + cl;
#pragma unroll
    for (int dy = 0; dy < TY + KS - 1; ++dy) {
      float vv[KS][2];
#pragma unroll
      for (int j = 0; j < KS; ++j) load2<BF16>(p, j * kSlice, vv[j]);
      p += rstride;
      // input row dy feeds output row r = dy - i through kernel row i
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int r = dy - i;
        if (r < 0 || r >= TY) continue;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          acc[r][0] = fmaf(wr[i * KS + j][0], vv[j][0], acc[r][0]);
          acc[r][1] = fmaf(wr[i * KS + j][1], vv[j][1], acc[r][1]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < TY; ++r) emit(y0 + r, x, slice * kSlice + cl, acc[r][0], acc[r][1]);
  }
}

// Stage the weights of channels [c0, c0 + nslices*32) into the sliced layout
// [slice][tap][32]: consecutive threads write consecutive words.  f_kk32
// divides by KS*KS*32.
template <int KS>
__device__ __forceinline__ void stage_weights(const float* __restrict__ w, int c0, int nslices,
                                              const FastDiv& f_kk32, float* Wt) {
  constexpr int KK = KS * KS;
  for (int d = threadIdx.x; d < KK * nslices * kSlice; d += kThreads) {
    const int slice = fdiv(d, f_kk32), rem = d - slice * (KK * kSlice);
    const int tap = rem / kSlice, cl = rem % kSlice;
    Wt[d] = w[(c0 + slice * kSlice + cl) * KK + tap];
  }
}

// Stage the zero-padded V tile (rows y0-P .., columns x0-P .., channels
// [c0, c0 + nslices*32)) and the matching weights into the sliced layouts.
template <bool BF16, int KS>
__device__ __forceinline__ void stage_halo(const void* __restrict__ Vimg,
                                           const float* __restrict__ w, const Shape& s,
                                           int y0, int x0, int hh, int hw, int c0, int nslices,
                                           const FastDiv& f_gs, const FastDiv& f_hw,
                                           const FastDiv& f_kk32, void* Hs, float* Wt) {
  using T = typename Elem<BF16>::T;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int GS = kSlice / VEC;               // 16-byte groups per pixel slice
  constexpr int P = KS / 2;
  const T* V = (const T*)Vimg;
  const int G = nslices * GS;                    // 16-byte groups per pixel
  const int ftop = y0 / s.Hf * s.Hf;             // first row of the region's frame
  for (int e = threadIdx.x; e < hh * hw * G; e += kThreads) {
    const int pix = fdiv(e, f_gs), g = e - pix * G;
    const int hy = fdiv(pix, f_hw), hx = pix - hy * hw;
    const int y = y0 + hy - P, x = x0 + hx - P;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (y >= ftop && y < ftop + s.Hf && x >= 0 && x < s.W)
      val = *(const uint4*)(V + (y * s.W + x) * s.C + c0 + g * VEC);
    const int slice = g / GS, gi = g - slice * GS;
    *(uint4*)((T*)Hs + ((slice * hh + hy) * hw + hx) * kSlice + gi * VEC) = val;
  }
  stage_weights<KS>(w, c0, nslices, f_kk32, Wt);
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
// once: K row-major [key][channel], V transposed [channel][key].  Each
// wavefront then runs its tasks over the chunk in steps of 32 keys with an
// online softmax:
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
// The softmax scale (positive) is folded into the exponent:
// p = 2^(s*c - m*c) with c = attn_scale*log2(e) and m the running row max.
//
// Epilogue (KS > 0): the region's zero-padded V halo tile (hs+KS-1 by
// ws+KS-1 pixels; loaded into registers before the attention loop when it
// is small enough, so that its latency hides behind the attention) and the
// LePE weights, both in the sliced layouts of conv_tile, and an fp32 tile
// L[pixel][channel] reuse the staging area; L is added to the normalised attention output before the
// single rounding to the output type.  With `accumulate` the kernel instead
// adds what `out` already holds (the LePE term written there first by the
// standalone kernel).
// ---------------------------------------------------------------------------
constexpr int kHeadDim = 32;
constexpr int kTasksPerWave = 2;
constexpr int kTasksPerBlock = kWaves * kTasksPerWave;
// Tuning constants (compile-time; the defaults are the measured best on
// MI355X for the BiFormer stage shapes).
#ifndef BRA_HALO_REGS
#define BRA_HALO_REGS 6                 // halo vectors per thread held in registers (0: off)
#endif
#ifndef BRA_STAGE_BATCH
#define BRA_STAGE_BATCH 2               // K/V vectors per thread loaded together
#endif
#ifndef BRA_KSTEP_MAX
#define BRA_KSTEP_MAX 64                // keys per softmax step (32 or 64)
#endif
#ifndef BRA_STREAM
#define BRA_STREAM 1                    // use the streaming kernel where it applies
#endif
#ifndef BRA_ATTN_WAVES_PER_SIMD
#define BRA_ATTN_WAVES_PER_SIMD 1       // occupancy the register allocator must allow
#endif
constexpr int kHaloRegs = BRA_HALO_REGS > 0 ? BRA_HALO_REGS : 1;
constexpr int kStageBatch = BRA_STAGE_BATCH;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  void* out;
  const float* w;       // fused LePE weights [C, KS, KS] (KS > 0)
  const float* bias;    // fused LePE bias [C] or null
  Shape s;
  float scale_log2;     // attn_scale * log2(e), > 0
  int kc;               // keys per LDS chunk (multiple of kStep)
  int krow;             // K LDS row stride in elements
  int vrow;             // V^T LDS row stride in elements (per channel)
  int lrow;             // L tile row stride in floats
  int groups;           // task groups (workgroups) per query region
  int units;            // B * R * groups
  int per_xcd;          // ceil(units / 8)
  int accumulate;       // add the existing contents of out
  int halo_pref;        // 1: prefetch the halo tile into registers
  int g_fixed;          // 1: the 16-byte groups per pixel divide the block
  int rbase_off;        // byte offset of the routed-region table in LDS
  FastDiv f_n, f_ws, f_S, f_G, f_heads, f_groups, f_R, f_hw, f_KK32, f_ns;
};

// 8 elements in MFMA operand slot order (bf16: one 8-wide vector).
template <bool BF16>
struct Operand;

template <>
struct Operand<true> {
  bf16x8 v;
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = __builtin_bit_cast(bf16x8, *(const uint4*)p);
  }
  // slots 0-3 from p0[0..3], slots 4-7 from p1[0..3]
  __device__ __forceinline__ void load_split(const uint16_t* p0, const uint16_t* p1) {
    const uint2 a = *(const uint2*)p0;
    const uint2 b = *(const uint2*)p1;
    v = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
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
  __device__ __forceinline__ void load_split(const float* p0, const float* p1) {
    const float4 a = *(const float4*)p0;
    const float4 b = *(const float4*)p1;
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

// key offset (within a 32-key half step) of operand slot e for lane group lg:
// slots 0-3 are keys 4*lg..4*lg+3, slots 4-7 keys 16+4*lg..16+4*lg+3, the
// rows a 16x16 MFMA output hands to lane group lg in its two key blocks.
__device__ __forceinline__ int slot_key(int lg, int e) {
  return e < 4 ? 4 * lg + e : 16 + 4 * lg + (e - 4);
}

template <bool BF16, int KS, int TY, int KSTEP>
__global__ __launch_bounds__(kThreads, BRA_ATTN_WAVES_PER_SIMD) void attend_kernel(AttnArgs A) {
  using T = typename Elem<BF16>::T;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int P = KS / 2;
  constexpr int NH = KSTEP / 32;                 // 32-key halves per step
  extern __shared__ uint4 smem_attn[];
  const Shape& s = A.s;

  // XCD-aware unit order: consecutive units (same image) land on one XCD.
  const int unit = (blockIdx.x % kXcds) * A.per_xcd + blockIdx.x / kXcds;
  if (unit >= A.units) return;
  const int br = fdiv(unit, A.f_groups);
  const int grp = unit - br * A.groups;
  const int b = fdiv(br, A.f_R), r = br - b * s.R;
  const int ry = fdiv(r, A.f_S), rx = r - ry * s.S;
  const size_t img = (size_t)b * s.H * s.W * s.C;

  T* Ks = (T*)smem_attn;                         // [kc][krow]
  T* Vt = Ks + A.kc * A.krow;                    // [C][vrow]
  int* rbase = (int*)((char*)smem_attn + A.rbase_off);   // [topk] region pixel offsets
  const T* __restrict__ Q = (const T*)A.q + img;
  const T* __restrict__ K = (const T*)A.k + img;
  const T* __restrict__ V = (const T*)A.v + img;
  const int G = s.C / VEC;                       // 16-byte groups per pixel
  // G divides the block: every vector a thread stages has the same group
  const int g_t = threadIdx.x % G, p_t = threadIdx.x / G, p_stride = kThreads / G;

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lq = lane & 15;     // query column of this lane / key row of an operand
  const int lg = lane >> 4;     // 0..3
  const int nqb = (s.n + 15) / 16;
  const int ntasks = nqb * s.heads;

  // routed regions -> element offset of their top-left pixel
  for (int j = threadIdx.x; j < s.topk; j += kThreads) {
    const int reg = min(max(A.idx[(size_t)br * s.topk + j], 0), s.R - 1);
    const int sy = fdiv(reg, A.f_S), sx = reg - sy * s.S;
    rbase[j] = (sy * s.hs * s.W + sx * s.ws) * s.C;
  }

  // per-task register state
  Operand<BF16> qop[kTasksPerWave];
  f32x4 acc0[kTasksPerWave], acc1[kTasksPerWave];
  float m_run[kTasksPerWave], l_run[kTasksPerWave];
  int t_head[kTasksPerWave], t_q[kTasksPerWave], t_pix[kTasksPerWave];
  bool t_ok[kTasksPerWave];
#pragma unroll
  for (int i = 0; i < kTasksPerWave; ++i) {
    const int task = grp * kTasksPerBlock + i * kWaves + wave;
    t_ok[i] = task < ntasks;
    const int qb = t_ok[i] ? fdiv(task, A.f_heads) : 0;
    t_head[i] = t_ok[i] ? task - qb * s.heads : 0;
    t_q[i] = qb * 16 + lq;                // query token index in the region
    const int ty = fdiv(t_q[i], A.f_ws), tx = t_q[i] - ty * s.ws;
    t_pix[i] = ((ry * s.hs + ty) * s.W + rx * s.ws + tx) * s.C;
    if (t_ok[i] && t_q[i] < s.n) {
      qop[i].load(Q + t_pix[i] + t_head[i] * kHeadDim + 8 * lg);
    } else {
      qop[i].zero();
    }
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }

  // halo prefetch (fused LePE): the zero-padded V tile around the region, in
  // registers until the attention is done; hoff[i] is its LDS destination
  const int hw = s.ws + KS - 1, hh = s.hs + KS - 1;
  uint4 hreg[KS > 0 ? kHaloRegs : 1];
  int hoffs[KS > 0 ? kHaloRegs : 1];
  if constexpr (KS > 0) {
    if (A.halo_pref) {
      constexpr int GS = kSlice / VEC;
      const int slice = g_t / GS, gi = g_t - slice * GS;
      const int hy0 = ry * s.hs - P, hx0 = rx * s.ws - P;
      const int ftop = ry * s.hs / s.Hf * s.Hf;   // first row of the region's frame
#pragma unroll
      for (int i = 0; i < kHaloRegs; ++i) {
        const int pix = p_t + i * p_stride;
        const int hy = fdiv(pix, A.f_hw), hx = pix - hy * hw;
        const int y = hy0 + hy, x = hx0 + hx;
        hreg[i] = make_uint4(0, 0, 0, 0);
        hoffs[i] = pix < hh * hw ? ((slice * hh + hy) * hw + hx) * kSlice + gi * VEC : -1;
        if (pix < hh * hw && y >= ftop && y < ftop + s.Hf && x >= 0 && x < s.W)
          hreg[i] = *(const uint4*)(V + (y * s.W + x) * s.C + g_t * VEC);
      }
    }
  }

  const float c = A.scale_log2;
  const int total = s.topk * s.n;
  bool first = true;
  for (int c0 = 0; c0 < total; c0 += A.kc) {
    const int kcnt = min(A.kc, total - c0);
    const int kpad = (kcnt + KSTEP - 1) / KSTEP * KSTEP;
    __syncthreads();
    // staging: batches of kStageBatch vectors per thread, all global loads of
    // a batch in flight before the first LDS write waits on them.  When G
    // does not divide the block, each vector works out its own group.
    if (!A.g_fixed) {
      for (int e = threadIdx.x; e < kpad * G; e += kThreads) {
        const int key = fdiv(e, A.f_G), g = e - key * G;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (key < kcnt) {
          const int t = c0 + key;
          const int j = fdiv(t, A.f_n), tok = t - j * s.n;
          const int ty = fdiv(tok, A.f_ws), tx = tok - ty * s.ws;
          const int off = rbase[j] + (ty * s.W + tx) * s.C + g * VEC;
          kv = *(const uint4*)(K + off);
          vv = *(const uint4*)(V + off);
        }
        *(uint4*)(Ks + key * A.krow + g * VEC) = kv;
        T* vt = Vt + (g * VEC) * A.vrow + key;
        float f[VEC];
        unpack16<BF16>(vv, f);
#pragma unroll
        for (int e2 = 0; e2 < VEC; ++e2) {
          if constexpr (BF16) {
            vt[e2 * A.vrow] = (uint16_t)(e2 & 1 ? ((&vv.x)[e2 / 2] >> 16) : ((&vv.x)[e2 / 2] & 0xffffu));
          } else {
            vt[e2 * A.vrow] = f[e2];
          }
        }
      }
    }
    for (int k0 = p_t; A.g_fixed && k0 < kpad; k0 += kStageBatch * p_stride) {
      uint4 kv[kStageBatch], vv[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int key = k0 + u * p_stride;
        kv[u] = make_uint4(0, 0, 0, 0);
        vv[u] = make_uint4(0, 0, 0, 0);
        if (key < kcnt) {
          const int t = c0 + key;
          const int j = fdiv(t, A.f_n), tok = t - j * s.n;
          const int ty = fdiv(tok, A.f_ws), tx = tok - ty * s.ws;
          const int off = rbase[j] + (ty * s.W + tx) * s.C + g_t * VEC;
          kv[u] = *(const uint4*)(K + off);
          vv[u] = *(const uint4*)(V + off);
        }
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int key = k0 + u * p_stride;
        if (key >= kpad) break;
        *(uint4*)(Ks + key * A.krow + g_t * VEC) = kv[u];
        // V transposed: element e of the vector is channel g*VEC + e
        T* vt = Vt + (g_t * VEC) * A.vrow + key;
        if constexpr (BF16) {
          vt[0 * A.vrow] = (uint16_t)(vv[u].x & 0xffffu); vt[1 * A.vrow] = (uint16_t)(vv[u].x >> 16);
          vt[2 * A.vrow] = (uint16_t)(vv[u].y & 0xffffu); vt[3 * A.vrow] = (uint16_t)(vv[u].y >> 16);
          vt[4 * A.vrow] = (uint16_t)(vv[u].z & 0xffffu); vt[5 * A.vrow] = (uint16_t)(vv[u].z >> 16);
          vt[6 * A.vrow] = (uint16_t)(vv[u].w & 0xffffu); vt[7 * A.vrow] = (uint16_t)(vv[u].w >> 16);
        } else {
          vt[0 * A.vrow] = __uint_as_float(vv[u].x); vt[1 * A.vrow] = __uint_as_float(vv[u].y);
          vt[2 * A.vrow] = __uint_as_float(vv[u].z); vt[3 * A.vrow] = __uint_as_float(vv[u].w);
        }
      }
    }
    __syncthreads();

    for (int ks = 0; ks < kpad; ks += KSTEP) {
      const bool tail = ks + KSTEP > kcnt;
#pragma unroll
      for (int i = 0; i < kTasksPerWave; ++i) {
        if (!t_ok[i]) continue;
        const int hoff = t_head[i] * kHeadDim;
        // S^T blocks: keys ks + 16*kb + lq as A rows, kb = 0 .. KSTEP/16-1
        float x[8 * NH];
#pragma unroll
        for (int kb = 0; kb < 2 * NH; ++kb) {
          Operand<BF16> ka;
          ka.load(Ks + (ks + 16 * kb + lq) * A.krow + hoff + 8 * lg);
          const f32x4 sv = mma(ka, qop[i], f32x4{0.f, 0.f, 0.f, 0.f});
          // lane holds keys ks + 16*kb + 4*lg + e of query lq
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * kb + e] = sv[e];
        }
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8 * NH; ++e)
            if (ks + 16 * (e / 4) + 4 * lg + (e & 3) >= kcnt) x[e] = -INFINITY;
        }
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8 * NH; ++e) mt = fmaxf(mt, x[e]);
        mt = fmaxf(mt, xor16(mt));
        mt = fmaxf(mt, xor32(mt));
        float mn = mt * c;                                // row max, scaled
        float alpha = 0.f;
        if (!first) {
          mn = fmaxf(m_run[i], mn);
          alpha = __builtin_amdgcn_exp2f(m_run[i] - mn);
        }
        m_run[i] = mn;
        float p[8 * NH];
#pragma unroll
        for (int e = 0; e < 8 * NH; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c, -mn));
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8 * NH; ++e) ps += p[e];
        if (!first) {
          l_run[i] = fmaf(l_run[i], alpha, ps);
          acc0[i] *= alpha;
          acc1[i] *= alpha;
        } else {
          l_run[i] = ps;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          // this half's keys: blocks 2h, 2h+1 -> P^T slots; p[8h + 4*half + e]
          const int kh = ks + 32 * h;
          const T* va_p = Vt + (hoff + lq) * A.vrow + kh + 4 * lg;
          const T* vb_p = va_p + 16 * A.vrow;
          Operand<BF16> va, vb;
          va.load_split(va_p, va_p + 16);
          vb.load_split(vb_p, vb_p + 16);
          const float* ph = p + 8 * h;
          if constexpr (BF16) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hi[e] = pack_bf16x2(ph[2 * e], ph[2 * e + 1]);
              lo[e] = pack_bf16x2(ph[2 * e] - bf16_lo(hi[e]), ph[2 * e + 1] - bf16_hi(hi[e]));
            }
            Operand<true> phi, plo;
            phi.v = as_bf16x8(hi[0], hi[1], hi[2], hi[3]);
            plo.v = as_bf16x8(lo[0], lo[1], lo[2], lo[3]);
            acc0[i] = mma(va, phi, acc0[i]);   // O^T rows d = 4*lg + e
            acc0[i] = mma(va, plo, acc0[i]);
            acc1[i] = mma(vb, phi, acc1[i]);   // O^T rows d = 16 + 4*lg + e
            acc1[i] = mma(vb, plo, acc1[i]);
          } else {
            Operand<false> pop;
#pragma unroll
            for (int e = 0; e < 8; ++e) pop.v[e] = ph[e];
            acc0[i] = mma(va, pop, acc0[i]);
            acc1[i] = mma(vb, pop, acc1[i]);
          }
        }
      }
      first = false;
    }
  }

  float* Ls = nullptr;
  if constexpr (KS > 0) {
    // fused LePE: sliced V halo tile, weights and the fp32 L tile in the
    // staging area
    const int nslices = s.C / kSlice;
    T* Hs = (T*)smem_attn;
    float* Wt = (float*)(Hs + hh * hw * s.C);
    Ls = Wt + KS * KS * s.C;
    __syncthreads();
    if (A.halo_pref) {
#pragma unroll
      for (int i = 0; i < kHaloRegs; ++i)
        if (hoffs[i] >= 0) *(uint4*)(Hs + hoffs[i]) = hreg[i];
      stage_weights<KS>(A.w, 0, nslices, A.f_KK32, Wt);
    } else {
      stage_halo<BF16, KS>(V, A.w, s, ry * s.hs, rx * s.ws, hh, hw, 0, nslices, A.f_G, A.f_hw,
                           A.f_KK32, Hs, Wt);
    }
    __syncthreads();
    conv_tile<BF16, KS, TY>(Hs, Wt, A.bias, 0, s.hs, s.ws, nslices, A.f_ws, A.f_ns,
        [&](int y, int x, int ch, float v0, float v1) {
          *(float2*)(Ls + (y * s.ws + x) * A.lrow + ch) = make_float2(v0, v1);
        });
    __syncthreads();
  }

  // normalise and store: lane holds query lq, channels 4*lg..+3 and 16+4*lg..+3
  T* out = (T*)A.out + img;
#pragma unroll
  for (int i = 0; i < kTasksPerWave; ++i) {
    if (!t_ok[i]) continue;
    float lt = l_run[i];
    lt += xor16(lt);
    lt += xor32(lt);
    if (t_q[i] >= s.n) continue;
    const float inv = 1.f / lt;
    const int o = t_pix[i] + t_head[i] * kHeadDim;
    float r0[4], r1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = acc0[i][e] * inv;
      r1[e] = acc1[i][e] * inv;
    }
    if constexpr (KS > 0) {
      const float* lp = Ls + t_q[i] * A.lrow + t_head[i] * kHeadDim;
      const float4 a0 = *(const float4*)(lp + 4 * lg);
      const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
      r0[0] += a0.x; r0[1] += a0.y; r0[2] += a0.z; r0[3] += a0.w;
      r1[0] += a1.x; r1[1] += a1.y; r1[2] += a1.z; r1[3] += a1.w;
    }
    if (A.accumulate) {
      float e0[4], e1[4];
      load4<BF16>(out, o + 4 * lg, e0);
      load4<BF16>(out, o + 16 + 4 * lg, e1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r0[e] += e0[e];
        r1[e] += e1[e];
      }
    }
    store4<BF16>(out, o + 4 * lg, r0);
    store4<BF16>(out, o + 16 + 4 * lg, r1);
  }
}

// ---------------------------------------------------------------------------
// Streaming variant of the fused gather-attention + LePE kernel for regions
// whose routed keys fit one LDS chunk (e.g. the BiFormer stage-1/2 shapes).
//
// A fixed set of workgroups (a few per CU) walks the query regions of its
// XCD's share, and software-pipelines them: while region u is computed, the
// global loads of region u+1 (its query operands and routed K/V vectors,
// addressed through a table of the workgroup's routing rows staged in LDS at
// start) and, once region u's halo has gone to LDS, region u+1's V halo are
// in flight in registers.  The LePE weights are staged once per workgroup.
// The arithmetic is that of attend_kernel; per region:
//   1. K/V vectors (registers) -> LDS, barrier
//   2. issue region u+1's Q and K/V loads
//   3. attention over the routed keys (MFMA, online softmax in one step)
//   4. barrier, halo vectors (registers) -> LDS, barrier; issue region
//      u+1's halo loads
//   5. LePE convolution -> fp32 L tile, barrier
//   6. normalise, add L, round once, store.
// ---------------------------------------------------------------------------
constexpr int kStreamHalo = 6;        // max halo vectors per thread per region

struct StreamArgs {
  AttnArgs a;
  int nhalo;            // halo vectors per thread (<= kStreamHalo)
  int blocks_per_xcd;   // workgroups per XCD
  int max_units;        // max regions per workgroup
  int wt_off, ls_off, idx_off;   // LDS byte offsets: weights, L tile, routing table
};

template <bool BF16, int KS, int TY, int KSTEP, int NKV>
__global__ __launch_bounds__(kThreads) void attend_stream_kernel(StreamArgs SA) {
  using T = typename Elem<BF16>::T;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int P = KS / 2;
  constexpr int NH = KSTEP / 32;
  constexpr int GS = kSlice / VEC;
  extern __shared__ uint4 smem_attn[];
  const AttnArgs& A = SA.a;
  const Shape& s = A.s;

  T* Ks = (T*)smem_attn;                         // [kc][krow]       (phase 1-3)
  T* Vt = Ks + A.kc * A.krow;                    // [C][vrow]        (phase 1-3)
  T* Hs = (T*)smem_attn;                         // halo tile        (phase 4-5)
  float* Wt = (float*)((char*)smem_attn + SA.wt_off);
  float* Ls = (float*)((char*)smem_attn + SA.ls_off);
  int* itab = (int*)((char*)smem_attn + SA.idx_off);    // [max_units][topk] routed region bases

  const int G = s.C / VEC;
  const int g_t = threadIdx.x % G, p_t = threadIdx.x / G, p_stride = kThreads / G;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lq = lane & 15, lg = lane >> 4;
  const int ntasks = ((s.n + 15) / 16) * s.heads;
  const int hw = s.ws + KS - 1, hh = s.hs + KS - 1;
  const int nslices = s.C / kSlice;
  const int total = s.topk * s.n;
  const int kpad = (total + KSTEP - 1) / KSTEP * KSTEP;
  const float c = A.scale_log2;

  // this workgroup's regions: u_k = base + k * stride, inside its XCD's range
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int ubase = xcd * A.per_xcd + slot, uend = min(A.units, (xcd + 1) * A.per_xcd);
  const int ustride = SA.blocks_per_xcd;
  const int nunits = ubase < uend ? (uend - ubase + ustride - 1) / ustride : 0;
  if (nunits == 0) return;

  // routing rows of all our regions -> element offsets of the routed regions
  for (int e = threadIdx.x; e < nunits * s.topk; e += kThreads) {
    const int k = e / s.topk, j = e - k * s.topk;
    const int u = ubase + k * ustride;
    const int reg = min(max(A.idx[(size_t)u * s.topk + j], 0), s.R - 1);
    const int sy = fdiv(reg, A.f_S), sx = reg - sy * s.S;
    itab[e] = (sy * s.hs * s.W + sx * s.ws) * s.C;
  }
  if constexpr (KS > 0) stage_weights<KS>(A.w, 0, nslices, A.f_KK32, Wt);
  __syncthreads();

  // register pipeline state
  Operand<BF16> qop[kTasksPerWave];
  uint4 kv[NKV], vv[NKV];
  uint4 hreg[KS > 0 ? kStreamHalo : 1];

  // task geometry (the same for every region)
  int t_head[kTasksPerWave], t_q[kTasksPerWave], t_rel[kTasksPerWave];
  bool t_ok[kTasksPerWave];
#pragma unroll
  for (int i = 0; i < kTasksPerWave; ++i) {
    const int task = i * kWaves + wave;
    t_ok[i] = task < ntasks;
    const int qb = t_ok[i] ? fdiv(task, A.f_heads) : 0;
    t_head[i] = t_ok[i] ? task - qb * s.heads : 0;
    t_q[i] = qb * 16 + lq;
    const int ty = fdiv(t_q[i], A.f_ws), tx = t_q[i] - ty * s.ws;
    t_rel[i] = (ty * s.W + tx) * s.C;          // query pixel relative to the region
  }
  // staged key geometry: key p_t + v * p_stride -> (routed region j, pixel offset)
  int k_j[NKV], k_rel[NKV];
#pragma unroll
  for (int v = 0; v < NKV; ++v) {
    const int key = p_t + v * p_stride;
    const int j = fdiv(key, A.f_n), tok = key - j * s.n;
    const int ty = fdiv(tok, A.f_ws), tx = tok - ty * s.ws;
    k_j[v] = j;
    k_rel[v] = (ty * s.W + tx) * s.C + g_t * VEC;
  }
  // halo geometry: pixel p_t + i * p_stride of the tile
  int h_dy[kStreamHalo], h_dx[kStreamHalo], h_lds[kStreamHalo];
  if constexpr (KS > 0) {
    const int slice = g_t / GS, gi = g_t - slice * GS;
#pragma unroll
    for (int i = 0; i < kStreamHalo; ++i) {
      const int pix = p_t + i * p_stride;
      const int hy = fdiv(pix, A.f_hw), hx = pix - hy * hw;
      h_dy[i] = hy - P;
      h_dx[i] = hx - P;
      h_lds[i] = ((slice * hh + hy) * hw + hx) * kSlice + gi * VEC;
    }
  }

  auto region_of = [&](int u, int& b, int& y0, int& x0) {
    b = fdiv(u, A.f_R);
    const int r = u - b * s.R;
    const int ry = fdiv(r, A.f_S), rx = r - ry * s.S;
    y0 = ry * s.hs;
    x0 = rx * s.ws;
  };
  auto load_qkv = [&](int k) {
    int b, y0, x0;
    region_of(ubase + k * ustride, b, y0, x0);
    const size_t img = (size_t)b * s.H * s.W * s.C;
    const T* Q = (const T*)A.q + img;
    const T* K = (const T*)A.k + img;
    const T* V = (const T*)A.v + img;
    const int rbase = (y0 * s.W + x0) * s.C;
#pragma unroll
    for (int i = 0; i < kTasksPerWave; ++i) {
      if (t_ok[i] && t_q[i] < s.n) qop[i].load(Q + rbase + t_rel[i] + t_head[i] * kHeadDim + 8 * lg);
      else qop[i].zero();
    }
#pragma unroll
    for (int v = 0; v < NKV; ++v) {
      kv[v] = make_uint4(0, 0, 0, 0);
      vv[v] = make_uint4(0, 0, 0, 0);
      if (p_t + v * p_stride < total) {
        const int off = itab[k * s.topk + k_j[v]] + k_rel[v];
        kv[v] = *(const uint4*)(K + off);
        vv[v] = *(const uint4*)(V + off);
      }
    }
  };
  auto load_halo = [&](int k) {
    int b, y0, x0;
    region_of(ubase + k * ustride, b, y0, x0);
    const T* V = (const T*)A.v + (size_t)b * s.H * s.W * s.C;
    const int ftop = y0 / s.Hf * s.Hf;           // first row of the region's frame
#pragma unroll
    for (int i = 0; i < kStreamHalo; ++i) {
      hreg[i] = make_uint4(0, 0, 0, 0);
      const int y = y0 + h_dy[i], x = x0 + h_dx[i];
      if (i < SA.nhalo && p_t + i * p_stride < hh * hw && y >= ftop && y < ftop + s.Hf &&
          x >= 0 && x < s.W)
        hreg[i] = *(const uint4*)(V + (y * s.W + x) * s.C + g_t * VEC);
    }
  };

  load_qkv(0);
  if constexpr (KS > 0) load_halo(0);

  for (int k = 0; k < nunits; ++k) {
    int b, y0, x0;
    region_of(ubase + k * ustride, b, y0, x0);
    // 1. K/V -> LDS
#pragma unroll
    for (int v = 0; v < NKV; ++v) {
      const int key = p_t + v * p_stride;
      if (key >= kpad) break;
      *(uint4*)(Ks + key * A.krow + g_t * VEC) = kv[v];
      T* vt = Vt + (g_t * VEC) * A.vrow + key;
      if constexpr (BF16) {
        vt[0 * A.vrow] = (uint16_t)(vv[v].x & 0xffffu); vt[1 * A.vrow] = (uint16_t)(vv[v].x >> 16);
        vt[2 * A.vrow] = (uint16_t)(vv[v].y & 0xffffu); vt[3 * A.vrow] = (uint16_t)(vv[v].y >> 16);
        vt[4 * A.vrow] = (uint16_t)(vv[v].z & 0xffffu); vt[5 * A.vrow] = (uint16_t)(vv[v].z >> 16);
        vt[6 * A.vrow] = (uint16_t)(vv[v].w & 0xffffu); vt[7 * A.vrow] = (uint16_t)(vv[v].w >> 16);
      } else {
        vt[0 * A.vrow] = __uint_as_float(vv[v].x); vt[1 * A.vrow] = __uint_as_float(vv[v].y);
        vt[2 * A.vrow] = __uint_as_float(vv[v].z); vt[3 * A.vrow] = __uint_as_float(vv[v].w);
      }
    }
    Operand<BF16> qcur[kTasksPerWave];
#pragma unroll
    for (int i = 0; i < kTasksPerWave; ++i) qcur[i] = qop[i];
    __syncthreads();
    // 2. next region's Q and K/V in flight during this one's compute
    if (k + 1 < nunits) load_qkv(k + 1);

    // 3. attention over all routed keys of this region
    f32x4 acc0[kTasksPerWave], acc1[kTasksPerWave];
    float m_run[kTasksPerWave], l_run[kTasksPerWave];
#pragma unroll
    for (int i = 0; i < kTasksPerWave; ++i) {
      acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[i] = -INFINITY;
      l_run[i] = 0.f;
    }
    for (int ks = 0; ks < kpad; ks += KSTEP) {
      const bool first = ks == 0, tail = ks + KSTEP > total;
#pragma unroll
      for (int i = 0; i < kTasksPerWave; ++i) {
        if (!t_ok[i]) continue;
        const int hoff = t_head[i] * kHeadDim;
        float x[8 * NH];
#pragma unroll
        for (int kb = 0; kb < 2 * NH; ++kb) {
          Operand<BF16> ka;
          ka.load(Ks + (ks + 16 * kb + lq) * A.krow + hoff + 8 * lg);
          const f32x4 sv = mma(ka, qcur[i], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * kb + e] = sv[e];
        }
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8 * NH; ++e)
            if (ks + 16 * (e / 4) + 4 * lg + (e & 3) >= total) x[e] = -INFINITY;
        }
        float mt = x[0];
#pragma unroll
        for (int e = 1; e < 8 * NH; ++e) mt = fmaxf(mt, x[e]);
        mt = fmaxf(mt, xor16(mt));
        mt = fmaxf(mt, xor32(mt));
        float mn = mt * c, alpha = 0.f;
        if (!first) {
          mn = fmaxf(m_run[i], mn);
          alpha = __builtin_amdgcn_exp2f(m_run[i] - mn);
        }
        m_run[i] = mn;
        float p[8 * NH];
#pragma unroll
        for (int e = 0; e < 8 * NH; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c, -mn));
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8 * NH; ++e) ps += p[e];
        if (!first) {
          l_run[i] = fmaf(l_run[i], alpha, ps);
          acc0[i] *= alpha;
          acc1[i] *= alpha;
        } else {
          l_run[i] = ps;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const T* va_p = Vt + (hoff + lq) * A.vrow + ks + 32 * h + 4 * lg;
          const T* vb_p = va_p + 16 * A.vrow;
          Operand<BF16> va, vb;
          va.load_split(va_p, va_p + 16);
          vb.load_split(vb_p, vb_p + 16);
          const float* ph = p + 8 * h;
          if constexpr (BF16) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hi[e] = pack_bf16x2(ph[2 * e], ph[2 * e + 1]);
              lo[e] = pack_bf16x2(ph[2 * e] - bf16_lo(hi[e]), ph[2 * e + 1] - bf16_hi(hi[e]));
            }
            Operand<true> phi, plo;
            phi.v = as_bf16x8(hi[0], hi[1], hi[2], hi[3]);
            plo.v = as_bf16x8(lo[0], lo[1], lo[2], lo[3]);
            acc0[i] = mma(va, phi, acc0[i]);
            acc0[i] = mma(va, plo, acc0[i]);
            acc1[i] = mma(vb, phi, acc1[i]);
            acc1[i] = mma(vb, plo, acc1[i]);
          } else {
            Operand<false> pop;
#pragma unroll
            for (int e = 0; e < 8; ++e) pop.v[e] = ph[e];
            acc0[i] = mma(va, pop, acc0[i]);
            acc1[i] = mma(vb, pop, acc1[i]);
          }
        }
      }
    }

    // 4-5. LePE of this region
    if constexpr (KS > 0) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kStreamHalo; ++i)
        if (i < SA.nhalo && p_t + i * p_stride < hh * hw) *(uint4*)(Hs + h_lds[i]) = hreg[i];
      __syncthreads();
      if (k + 1 < nunits) load_halo(k + 1);
      conv_tile<BF16, KS, TY>(Hs, Wt, A.bias, 0, s.hs, s.ws, nslices, A.f_ws, A.f_ns,
          [&](int y, int x, int ch, float v0, float v1) {
            *(float2*)(Ls + (y * s.ws + x) * A.lrow + ch) = make_float2(v0, v1);
          });
      __syncthreads();
    }

    // 6. normalise, add L, round once, store
    T* out = (T*)A.out + (size_t)b * s.H * s.W * s.C + (y0 * s.W + x0) * s.C;
#pragma unroll
    for (int i = 0; i < kTasksPerWave; ++i) {
      if (!t_ok[i]) continue;
      float lt = l_run[i];
      lt += xor16(lt);
      lt += xor32(lt);
      if (t_q[i] >= s.n) continue;
      const float inv = 1.f / lt;
      const int o = t_rel[i] + t_head[i] * kHeadDim;
      float r0[4], r1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r0[e] = acc0[i][e] * inv;
        r1[e] = acc1[i][e] * inv;
      }
      if constexpr (KS > 0) {
        const float* lp = Ls + t_q[i] * A.lrow + t_head[i] * kHeadDim;
        const float4 a0 = *(const float4*)(lp + 4 * lg);
        const float4 a1 = *(const float4*)(lp + 16 + 4 * lg);
        r0[0] += a0.x; r0[1] += a0.y; r0[2] += a0.z; r0[3] += a0.w;
        r1[0] += a1.x; r1[1] += a1.y; r1[2] += a1.z; r1[3] += a1.w;
      }
      store4<BF16>(out, o + 4 * lg, r0);
      store4<BF16>(out, o + 16 + 4 * lg, r1);
    }
    if constexpr (KS == 0) __syncthreads();   // K/V area is rewritten next
  }
}

// ---------------------------------------------------------------------------
// Standalone LePE: out = L (ACCUM false) or out += L (ACCUM true), L as in
// conv_tile.  One workgroup per output tile of kLepeRows rows by kLepeCols
// columns and one slice of up to 64 channels; the zero-padded V tile (zeros
// also past the image edge) and the slice's weights are staged in LDS with
// 16-byte loads, then convolved.
// ---------------------------------------------------------------------------
constexpr int kLepeRows = 8;
constexpr int kLepeCols = 16;

struct LepeArgs {
  const void* v;
  const float* w;
  const float* bias;
  void* out;
  Shape s;
  int cs;        // channels per slice (64 or 32)
  int tiles_y;   // row tiles per image
  FastDiv f_g, f_hw, f_kk, f_tw, f_ns;
};

template <bool BF16, int KS, bool ACCUM>
__global__ __launch_bounds__(kThreads) void lepe_kernel(LepeArgs A) {
  using T = typename Elem<BF16>::T;
  constexpr int HW = kLepeCols + KS - 1, HH = kLepeRows + KS - 1;
  extern __shared__ uint4 smem_lepe[];
  const Shape& s = A.s;
  const int cs = A.cs;
  const int c0 = blockIdx.z * cs;
  const int x0 = blockIdx.x * kLepeCols;
  const int b = blockIdx.y / A.tiles_y;
  const int y0 = (blockIdx.y - b * A.tiles_y) * kLepeRows;
  const size_t img = (size_t)b * s.H * s.W * s.C;
  const T* __restrict__ V = (const T*)A.v + img;
  T* Hs = (T*)smem_lepe;
  float* Wt = (float*)(Hs + HH * HW * cs);
  const int nslices = cs / kSlice;
  stage_halo<BF16, KS>(V, A.w, s, y0, x0, HH, HW, c0, nslices, A.f_g, A.f_hw, A.f_kk, Hs, Wt);
  __syncthreads();
  T* out = (T*)A.out + img;
  conv_tile<BF16, KS, kLepeRows>(Hs, Wt, A.bias, c0, kLepeRows, kLepeCols, nslices, A.f_tw,
                                 A.f_ns,
      [&](int y, int x, int c, float v0, float v1) {
        if (y0 + y >= s.H || x0 + x >= s.W) return;
        const int off = ((y0 + y) * s.W + x0 + x) * s.C + c0 + c;
        if constexpr (ACCUM) {
          float e[2];
          load2<BF16>(out, off, e);
          v0 += e[0];
          v1 += e[1];
        }
        store2<BF16>(out, off, v0, v1);
      });
}

template <bool BF16, int KS, bool ACCUM>
hipError_t lepe_launch_ks(const void* v, const float* w, const float* b, const Shape& s,
                          void* out, hipStream_t st) {
  LepeArgs a;
  a.v = v; a.w = w; a.bias = b; a.out = out; a.s = s;
  a.cs = (s.C % 64 == 0) ? 64 : 32;
  a.tiles_y = (s.H + kLepeRows - 1) / kLepeRows;
  const int vec = BF16 ? 8 : 4;
  a.f_g = make_fastdiv(a.cs / vec);
  a.f_hw = make_fastdiv(kLepeCols + KS - 1);
  a.f_kk = make_fastdiv(KS * KS * kSlice);
  a.f_tw = make_fastdiv(kLepeCols);
  a.f_ns = make_fastdiv(a.cs / kSlice);
  const dim3 grid((unsigned)((s.W + kLepeCols - 1) / kLepeCols), (unsigned)(s.B * a.tiles_y),
                  (unsigned)(s.C / a.cs));
  const size_t esz = BF16 ? 2 : 4;
  const size_t lds = (size_t)(kLepeRows + KS - 1) * (kLepeCols + KS - 1) * a.cs * esz +
                     (size_t)KS * KS * a.cs * sizeof(float);
  const void* fn = (const void*)lepe_kernel<BF16, KS, ACCUM>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lepe_kernel<BF16, KS, ACCUM>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <bool BF16, bool ACCUM>
hipError_t lepe_launch(const void* v, const float* w, const float* b, int ks, const Shape& s0,
                       void* out, hipStream_t st) {
  // LePE is per frame: a clip of H / Hf stacked frames is a batch of frames
  Shape s = s0;
  if (s0.Hf < 1 || s0.H % s0.Hf) return hipErrorInvalidValue;
  s.B = s0.B * (s0.H / s0.Hf);
  s.H = s0.Hf;
  switch (ks) {
    case 1: return lepe_launch_ks<BF16, 1, ACCUM>(v, w, b, s, out, st);
    case 3: return lepe_launch_ks<BF16, 3, ACCUM>(v, w, b, s, out, st);
    case 5: return lepe_launch_ks<BF16, 5, ACCUM>(v, w, b, s, out, st);
    case 7: return lepe_launch_ks<BF16, 7, ACCUM>(v, w, b, s, out, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int KS, int TY, int KSTEP, int NKV>
hipError_t stream_launch_nkv(const StreamArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const void* fn = (const void*)attend_stream_kernel<BF16, KS, TY, KSTEP, NKV>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_stream_kernel<BF16, KS, TY, KSTEP, NKV>), grid, dim3(kThreads), lds,
                     st, a);
  return hipGetLastError();
}

template <bool BF16, int KS, int TY, int KSTEP>
hipError_t stream_launch_step(const StreamArgs& a, int nkv, dim3 grid, size_t lds, hipStream_t st) {
  switch (nkv) {
    case 1: return stream_launch_nkv<BF16, KS, TY, KSTEP, 1>(a, grid, lds, st);
    case 2: return stream_launch_nkv<BF16, KS, TY, KSTEP, 2>(a, grid, lds, st);
    case 4: return stream_launch_nkv<BF16, KS, TY, KSTEP, 4>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int KS, int TY>
hipError_t stream_launch_ty(const StreamArgs& a, int kstep, int nkv, dim3 grid, size_t lds,
                            hipStream_t st) {
  return kstep == 64 ? stream_launch_step<BF16, KS, TY, 64>(a, nkv, grid, lds, st)
                     : stream_launch_step<BF16, KS, TY, 32>(a, nkv, grid, lds, st);
}

template <bool BF16>
hipError_t stream_launch(const StreamArgs& a, int ks, int ty, int kstep, int nkv, dim3 grid,
                         size_t lds, hipStream_t st) {
  if (ks == 0) return stream_launch_ty<BF16, 0, 1>(a, kstep, nkv, grid, lds, st);
#define BRA_KS_TY(KS_)                                                              \
  if (ks == KS_) {                                                                  \
    switch (ty) {                                                                   \
      case 1: return stream_launch_ty<BF16, KS_, 1>(a, kstep, nkv, grid, lds, st);  \
      case 2: return stream_launch_ty<BF16, KS_, 2>(a, kstep, nkv, grid, lds, st);  \
      case 4: return stream_launch_ty<BF16, KS_, 4>(a, kstep, nkv, grid, lds, st);  \
      case 8: return stream_launch_ty<BF16, KS_, 8>(a, kstep, nkv, grid, lds, st);  \
      default: return hipErrorInvalidValue;                                         \
    }                                                                               \
  }
  BRA_KS_TY(1) BRA_KS_TY(3) BRA_KS_TY(5) BRA_KS_TY(7)
#undef BRA_KS_TY
  return hipErrorInvalidValue;
}

template <bool BF16, int KS, int TY, int KSTEP>
hipError_t attend_launch_ks(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const void* fn = (const void*)attend_kernel<BF16, KS, TY, KSTEP>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_kernel<BF16, KS, TY, KSTEP>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <bool BF16, int KS, int TY>
hipError_t attend_launch_step(const AttnArgs& a, int kstep, dim3 grid, size_t lds,
                              hipStream_t st) {
  return kstep == 64 ? attend_launch_ks<BF16, KS, TY, 64>(a, grid, lds, st)
                     : attend_launch_ks<BF16, KS, TY, 32>(a, grid, lds, st);
}

template <bool BF16, int KS>
hipError_t attend_launch_ty(const AttnArgs& a, int ty, int kstep, dim3 grid, size_t lds,
                            hipStream_t st) {
  switch (ty) {
    case 1: return attend_launch_step<BF16, KS, 1>(a, kstep, grid, lds, st);
    case 2: return attend_launch_step<BF16, KS, 2>(a, kstep, grid, lds, st);
    case 4: return attend_launch_step<BF16, KS, 4>(a, kstep, grid, lds, st);
    case 8: return attend_launch_step<BF16, KS, 8>(a, kstep, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
hipError_t attend_launch(const AttnArgs& a, int ks, int ty, int kstep, dim3 grid, size_t lds,
                         hipStream_t st) {
  switch (ks) {
    case 0: return attend_launch_step<BF16, 0, 1>(a, kstep, grid, lds, st);
    case 1: return attend_launch_ty<BF16, 1>(a, ty, kstep, grid, lds, st);
    case 3: return attend_launch_ty<BF16, 3>(a, ty, kstep, grid, lds, st);
    case 5: return attend_launch_ty<BF16, 5>(a, ty, kstep, grid, lds, st);
    case 7: return attend_launch_ty<BF16, 7>(a, ty, kstep, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attend(const void* q, const void* k, const void* v, const int32_t* idx,
                         const Shape& s, bool bf16, float attn_scale, const float* w,
                         const float* bias, int ks, void* out, hipStream_t st) {
  if (bf16 && w) {
    // a shape with its own kernel runs there: whole image in LDS first, then
    // the per-region gather
    hipError_t e = launch_attend_image(q, k, v, idx, s, attn_scale, w, bias, ks, out, st);
    if (e != hipErrorNotSupported) return e;
    e = launch_attend_region(q, k, v, idx, s, attn_scale, w, bias, ks, out, st);
    if (e != hipErrorNotSupported) return e;
  }
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.idx = idx; a.out = out; a.w = w; a.bias = bias; a.s = s;
  a.scale_log2 = attn_scale * 1.4426950408889634f;
  a.accumulate = 0;
  a.halo_pref = 0;
  const int esz = bf16 ? 2 : 4;
  const int vec = 16 / esz;
  a.krow = s.C + vec;                                    // 16-byte pad per K row
  a.lrow = s.C + 4;
  const size_t budget = 64 * 1024;
  const int total = s.topk * s.n;
  // keys per step: 64 when a chunk can hold a multiple of 64 keys
  const int per_key = (a.krow + s.C) * esz;   // one K row + one V^T column
  const int kmax = (int)(budget / (size_t)per_key);
  const int kstep = (BRA_KSTEP_MAX >= 64 && kmax >= 64 && total > 32) ? 64 : 32;
  int kc = kmax / kstep * kstep;
  if (kc < kstep) kc = kstep;
  const int total_pad = (total + kstep - 1) / kstep * kstep;
  if (kc > total_pad) kc = total_pad;
  a.kc = kc;
  a.vrow = kc + 4;                                       // pad per V^T row
  const int ntasks = ((s.n + 15) / 16) * s.heads;
  a.groups = (ntasks + kTasksPerBlock - 1) / kTasksPerBlock;
  a.units = s.B * s.R * a.groups;
  a.per_xcd = (a.units + kXcds - 1) / kXcds;
  const int G = s.C / vec;
  a.g_fixed = (kThreads % G == 0) ? 1 : 0;
  a.f_n = make_fastdiv(s.n);
  a.f_ws = make_fastdiv(s.ws);
  a.f_S = make_fastdiv(s.S);
  a.f_G = make_fastdiv(G);
  a.f_heads = make_fastdiv(s.heads);
  a.f_groups = make_fastdiv(a.groups);
  a.f_R = make_fastdiv(s.R);
  a.f_ns = make_fastdiv(s.C / kSlice);
  size_t main_lds = (size_t)kc * a.krow * esz + (size_t)s.C * a.vrow * esz;
  const dim3 grid((unsigned)(a.per_xcd * kXcds));
  int fused_ks = 0, ty = 1;
  if (w) {
    a.f_hw = make_fastdiv(s.ws + ks - 1);
    a.f_KK32 = make_fastdiv(ks * ks * kSlice);
    const size_t hpix = (size_t)(s.hs + ks - 1) * (s.ws + ks - 1);
    const size_t halo = hpix * s.C * esz + (size_t)ks * ks * s.C * sizeof(float) +
                        (size_t)s.n * a.lrow * sizeof(float);
    if (a.groups == 1 && halo <= (main_lds > budget ? main_lds : budget)) {
      fused_ks = ks;
      ty = s.hs % 8 == 0 ? 8 : s.hs % 4 == 0 ? 4 : s.hs % 2 == 0 ? 2 : 1;
      // prefetch: each thread holds the halo pixels p_t + i * (256 / G)
      a.halo_pref = (BRA_HALO_REGS > 0 && a.g_fixed &&
                     hpix <= (size_t)kHaloRegs * (kThreads / G)) ? 1 : 0;
      if (halo > main_lds) main_lds = halo;
    } else {
      // LePE first (out = L), then attention adds its result into out
      const hipError_t e = bf16 ? lepe_launch<true, false>(v, w, bias, ks, s, out, st)
                                : lepe_launch<false, false>(v, w, bias, ks, s, out, st);
      if (e != hipSuccess) return e;
      a.accumulate = 1;
    }
  }
  // Streaming path: one chunk holds all routed keys, the LePE (if any) is
  // fused, the staging vectors of a thread fit its register pipeline.
  {
    const int kpad = (total + kstep - 1) / kstep * kstep;
    const int p_stride = kThreads / G;
    const int nkv = (kpad + p_stride - 1) / p_stride;
    const int hpix = w ? (s.hs + ks - 1) * (s.ws + ks - 1) : 0;
    const int nhalo = (hpix + p_stride - 1) / p_stride;
    const bool fits = a.g_fixed && a.groups == 1 && !a.accumulate && kpad <= kc &&
                      (nkv == 1 || nkv == 2 || nkv == 4) && nhalo <= kStreamHalo &&
                      (w == nullptr || fused_ks == ks);
    if (fits && BRA_STREAM) {
      StreamArgs sa;
      sa.a = a;
      sa.nhalo = nhalo;
      const size_t r1 = main_lds > (size_t)0 ? main_lds : 0;   // K/V or halo, whichever is larger
      const size_t kvb = (size_t)kc * a.krow * esz + (size_t)s.C * a.vrow * esz;
      const size_t hb = (size_t)hpix * s.C * esz;
      size_t off = ((kvb > hb ? kvb : hb) + 15) / 16 * 16;
      (void)r1;
      sa.wt_off = (int)off;
      off += (size_t)ks * ks * s.C * sizeof(float) * (w ? 1 : 0);
      off = (off + 15) / 16 * 16;
      sa.ls_off = (int)off;
      off += (size_t)s.n * a.lrow * sizeof(float) * (w ? 1 : 0);
      off = (off + 15) / 16 * 16;
      sa.idx_off = (int)off;
      // workgroups per CU from the LDS footprint (a few KB left for the table)
      const size_t base_lds = off + 4096;
      int bpc = (int)((160 * 1024) / base_lds);
      if (bpc > 4) bpc = 4;
      if (bpc < 1) bpc = 1;
      // launches over image ranges that keep the routing table within
      // kTableBytes (at least 32 workgroups per XCD)
      const long long upi = (long long)s.R * a.groups;
      const int per = images_per_launch(s.B, upi, kXcds, 1, 32, s.topk, kTableBytes);
      if (per >= 1) {
        const size_t img_bytes = (size_t)s.H * s.W * s.C * esz;
        for (int b0 = 0; b0 < s.B; b0 += per) {
          const int nb = s.B - b0 < per ? s.B - b0 : per;
          StreamArgs c = sa;
          c.a.q = (const char*)q + b0 * img_bytes;
          c.a.k = (const char*)k + b0 * img_bytes;
          c.a.v = (const char*)v + b0 * img_bytes;
          c.a.out = (char*)out + b0 * img_bytes;
          c.a.idx = idx + (size_t)b0 * s.R * s.topk;
          c.a.s.B = nb;
          c.a.units = (int)(nb * upi);
          c.a.per_xcd = (int)units_per_xcd(c.a.units, kXcds, 1);
          int bpx = 32 * bpc;                       // 32 CUs per XCD
          if (bpx > c.a.per_xcd) bpx = c.a.per_xcd;
          c.blocks_per_xcd = bpx;
          c.max_units = (int)units_per_workgroup(c.a.per_xcd, bpx);
          const size_t lds = off + (size_t)c.max_units * s.topk * sizeof(int);
          const dim3 sgrid((unsigned)(bpx * kXcds));
          const hipError_t e = bf16 ? stream_launch<true>(c, fused_ks, ty, kstep, nkv, sgrid, lds, st)
                                    : stream_launch<false>(c, fused_ks, ty, kstep, nkv, sgrid, lds, st);
          if (e != hipSuccess) return e;
        }
        return hipSuccess;
      }
    }
  }
  main_lds = (main_lds + 15) / 16 * 16;
  a.rbase_off = (int)main_lds;
  const size_t lds = main_lds + (size_t)s.topk * sizeof(int);
  return bf16 ? attend_launch<true>(a, fused_ks, ty, kstep, grid, lds, st)
              : attend_launch<false>(a, fused_ks, ty, kstep, grid, lds, st);
}

hipError_t launch_lepe(const void* v, const float* w, const float* b, int ks, const Shape& s,
                       bool bf16, void* out, hipStream_t st) {
  return bf16 ? lepe_launch<true, true>(v, w, b, ks, s, out, st)
              : lepe_launch<false, true>(v, w, b, ks, s, out, st);
}

}  // namespace bra
