// gfx950 kernels of the bounded-KV block attention path.
//
//   rope_table_kernel  (cos, sin) tables of the 3D RoPE, computed in fp64
//   open_kernel        block open: store the pose, cosine top-k over the bank
//                      (fp64, one thread per candidate, ties to the lower
//                      stream id), and the current block's temporal RoPE rows
//   append_kernel      K with fused 3D RoPE -> cache rows; V -> cache V^T
//   append_k8_kernel   the same with K stored as E4M3 + per-tile exponents
//                      (and, for the FP8 KV cache, V^T as E4M3 too)
//   qkv_gemm_kernel    fused QKV projection (bf16 MFMA) with the append's
//                      epilogue: q to scratch, K rotated into the cache, V^T
//   attn_bf16_kernel   flash attention on bf16 MFMA (32x32x16), K/V tiles
//                      staged in LDS, online softmax in fp32; with an FP8
//                      key cache Q K^T runs on scaled E4M3 MFMA (32x32x64)
//   attn_merge_kernel  split launch: combines the key parts of the cut units
//   attn_f32_kernel    the same contraction in fp32 on the vector ALUs
//   gather_kernel      ConvKV and context-relative positions: raw K of the
//                      context's cached segments -> context-K rows, rotated
//                      at context positions
//   gather_k8_kernel   the same into E4M3 rows + per-tile exponents
//   conv_kernel        ConvKV: depthwise temporal conv of evicted frames
//   vquant_kernel      FP8 KV cache, ConvKV memory: bf16 V^T -> E4M3 V^T
//   export_kernel      inspection copy of one context segment
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.hpp"

namespace bkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// Rotate the channel pair (ch, ch+1) of a token at (t-table row, y, x).
__device__ __forceinline__ void rope_pair(float& u0, float& u1, int ch, const Rope& r, int trow,
                                          int y, int x) {
  float2 cs;
  if (ch < r.dt) {
    cs = r.t[trow * (r.dt >> 1) + (ch >> 1)];
  } else if (ch < r.dt + r.dh) {
    cs = r.h[y * (r.dh >> 1) + ((ch - r.dt) >> 1)];
  } else {
    cs = r.w[x * (r.dw >> 1) + ((ch - r.dt - r.dh) >> 1)];
  }
  const float a = u0 * cs.x - u1 * cs.y;
  const float b = u0 * cs.y + u1 * cs.x;
  u0 = a;
  u1 = b;
}

// The (cos, sin) of the channel pair (ch, ch+1), with the table picked by
// selects rather than branches, so that lanes whose channels fall on
// different axes issue one load each instead of taking the three paths in
// turn, and no load sits in a branch.  The three tables are addressed from
// the t table with uniform element offsets, so the selects choose an index,
// never a kernel-argument field (which the compiler would turn into a
// per-lane load of the argument ahead of the table load).  rope_rot applies
// the pair.
struct RopeSel {
  const float2* base;
  long long oh, ow;
  int dt, dth, ht, hh, hw;
  __device__ explicit RopeSel(const Rope& r)
      : base(r.t), oh(r.h - r.t), ow(r.w - r.t), dt(r.dt), dth(r.dt + r.dh), ht(r.dt >> 1),
        hh(r.dh >> 1), hw(r.dw >> 1) {}
  __device__ __forceinline__ float2 cs(int ch, int trow, int y, int x) const {
    const bool in_t = ch < dt, in_h = ch < dth;
    const float2* tab = base + (in_t ? 0 : (in_h ? oh : ow));
    const int idx = in_t ? trow * ht + (ch >> 1) : (in_h ? y * hh + ((ch - dt) >> 1) : x * hw + ((ch - dth) >> 1));
    return tab[idx];
  }
};

__device__ __forceinline__ void rope_rot(float& u0, float& u1, float2 cs) {
  const float a = u0 * cs.x - u1 * cs.y;
  const float b = u0 * cs.y + u1 * cs.x;
  u0 = a;
  u1 = b;
}

__device__ __forceinline__ bool has_rope(const Rope& r) { return (r.dt + r.dh + r.dw) != 0; }

// token index within a block -> (frame, y, x)
__device__ __forceinline__ void token_fyx(int tok, int gh, int gw, int& f, int& y, int& x) {
  const int per = gh * gw;
  f = tok / per;
  const int rem = tok - f * per;
  y = rem / gw;
  x = rem - y * gw;
}

// ------------------------------------------------------------------ tables
__global__ void rope_table_kernel(float2* tab, int rows, int half, int dim, long long pos0,
                                  double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * half) return;
  const int r = idx / half, i = idx - r * half;
  const double w = pow(theta, -2.0 * (double)i / (double)dim);
  const double phi = (double)(pos0 + r) * w;
  double s, c;
  sincos(phi, &s, &c);
  tab[idx] = make_float2((float)c, (float)s);
}

// ------------------------------------------------------------------ block open
// 256 threads, one per bank candidate.  Scores: cos = dot / (sqrt(|q|^2)
// sqrt(|b|^2)) in fp64, each candidate's sums in one fixed sequential order
// over the pose dimensions (staged through LDS 64 dimensions at a time, rows
// padded so that the 256 lanes hit distinct banks); 0 when either norm is 0
// or the score is not finite (a pose holding Inf or NaN), so every candidate
// has a finite score and each rank round has a winner.
// Rank: (score desc, stream id asc), k rounds of an arg-max by wave 0.
// Staging: each thread issues kOpenBatch pose loads before it writes any of
// them to LDS (indices past the end load the last element again).
constexpr int kOpenThreads = 256;
constexpr int kOpenChunk = 64;
constexpr int kOpenBatch = 4;
__global__ __launch_bounds__(kOpenThreads) void open_kernel(OpenArgs a) {
  __shared__ double s_score[kMaxBank];
  __shared__ int s_taken[kMaxBank];
  __shared__ int s_slot[kMaxBank];
  __shared__ int s_id[kMaxBank];
  __shared__ float s_q[kOpenChunk];
  __shared__ float s_b[kMaxBank][kOpenChunk + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < a.nbank) {
    s_slot[tid] = a.bank_dev ? a.bank_dev[kMaxBank + tid] : a.bank_slot[tid];
    s_id[tid] = a.bank_dev ? a.bank_dev[tid] : a.bank_id[tid];
  }
  if (a.bank_dev && a.upd_pos >= 0 && tid == 0) {   // a block joins a bank with room
    a.bank_dev[a.upd_pos] = a.upd_id;
    a.bank_dev[kMaxBank + a.upd_pos] = a.upd_slot;
  }
  if (a.pose_in) {
    for (int i = tid; i < a.P; i += kOpenThreads) a.pose_store[(size_t)a.cur_slot * a.P + i] = a.pose_in[i];
  }
  // the block's temporal RoPE rows: (cos, sin) of (t_pos0 + r) * theta^(-2i/t_dim)
  auto write_ttab = [&](int first, int stride) {
    if (!a.ttab) return;
    const int half = a.t_dim >> 1;
    for (int idx = first; idx < a.t_rows * half; idx += stride) {
      const int r = idx / half, i = idx - r * half;
      const double w = pow(a.theta, -2.0 * (double)i / (double)a.t_dim);
      double sn, cs;
      sincos((double)(a.t_pos0 + r) * w, &sn, &cs);
      a.ttab[idx] = make_float2((float)cs, (float)sn);
    }
  };
  if (a.k <= 0 || a.nbank <= 0) {
    write_ttab(tid, kOpenThreads);
    return;
  }
  const int nb = a.nbank;
  const float* qsrc = a.query ? a.query : a.pose_in;
  double qq = 0.0, dot = 0.0, bb = 0.0;
  for (int c0 = 0; c0 < a.P; c0 += kOpenChunk) {
    const int w = min(kOpenChunk, a.P - c0);
    __syncthreads();                       // the previous chunk has been consumed
    if (tid < w) s_q[tid] = qsrc[c0 + tid];
    const int n = nb * w;
    for (int base = 0; base < n; base += kOpenBatch * kOpenThreads) {
      float v[kOpenBatch];
#pragma unroll
      for (int u = 0; u < kOpenBatch; ++u) {
        const int idx = min(base + u * kOpenThreads + tid, n - 1);
        const int c = idx / w, i = idx - c * w;
        v[u] = a.pose_store[(size_t)s_slot[c] * a.P + c0 + i];
      }
#pragma unroll
      for (int u = 0; u < kOpenBatch; ++u) {
        const int idx = base + u * kOpenThreads + tid;
        if (idx < n) {
          const int c = idx / w, i = idx - c * w;
          s_b[c][i] = v[u];
        }
      }
    }
    __syncthreads();
    if (tid < nb) {
      for (int i = 0; i < w; ++i) {
        const double x = (double)s_q[i];
        const double y = (double)s_b[tid][i];
        qq += x * x;
        dot += x * y;
        bb += y * y;
      }
    }
  }
  if (tid < nb) {
    double sc = 0.0;
    if (qq > 0.0 && bb > 0.0) sc = dot / (sqrt(qq) * sqrt(bb));
    if (!isfinite(sc)) sc = 0.0;
    s_score[tid] = sc;
    s_taken[tid] = 0;
  }
  __syncthreads();
  if (tid >= 64) {                       // waves 1-3 write the RoPE rows while wave 0 ranks
    write_ttab(tid - 64, kOpenThreads - 64);
    return;
  }
  const int kk = a.k < nb ? a.k : nb;
  for (int r = 0; r < kk; ++r) {
    double best = -INFINITY;
    int bid = 0x7fffffff, bc = -1;
    for (int c = lane; c < nb; c += 64) {
      if (s_taken[c]) continue;
      const double sc = s_score[c];
      const int id = s_id[c];
      if (sc > best || (sc == best && id < bid)) {
        best = sc;
        bid = id;
        bc = c;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int oid = __shfl_xor(bid, off);
      const int oc = __shfl_xor(bc, off);
      if (ob > best || (ob == best && oid < bid)) {
        best = ob;
        bid = oid;
        bc = oc;
      }
    }
    if (lane == 0) {
      a.sel_ids[r] = bid;
      a.sel_slots[r] = s_slot[bc];
      s_taken[bc] = 1;
      if (a.victim_out) {                  // replacement: the first-ranked member leaves the bank
        a.victim_out[0] = bid;
        a.victim_out[1] = s_slot[bc];
        a.bank_dev[bc] = a.upd_id;
        a.bank_dev[kMaxBank + bc] = a.upd_slot;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
}

// ------------------------------------------------------------------ append
// V^T rows of one (64-token tile, head) from the token-major V tile in LDS
// (16-byte chunk c of row r at c ^ ((r >> 3) & 7)): each thread reads 8-byte
// slices of TOK consecutive tokens and writes CH rows of V^T (TOK tokens of
// one channel, 16 bytes each); consecutive lanes take consecutive token
// groups, so each V^T row is written in contiguous runs.  Tokens past the
// block's end are never written, so the V^T pad columns keep their zeros.
template <typename T, int D>
__device__ __forceinline__ void store_vt(const AppendArgs& a, const char* s_v, int tile0, int head,
                                         int ntok) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RS = D * (int)sizeof(T);
  constexpr int CH = 8 / sizeof(T);
  constexpr int TOK = VEC;
  const int tid = threadIdx.x;
  constexpr int NCG = D / CH, NTG = 64 / TOK;  // channel groups, token groups
  for (int task = tid; task < NCG * NTG; task += 256) {
    const int tg = task % NTG, cg = task / NTG;
    const int t0 = tg * TOK;
    if (t0 >= ntok) continue;
    typedef T rowv __attribute__((ext_vector_type(TOK)));
    typedef T slicev __attribute__((ext_vector_type(CH)));
    rowv col[CH];
#pragma unroll
    for (int e = 0; e < TOK; ++e) {
      const int t = t0 + e;
      const slicev w = *reinterpret_cast<const slicev*>(s_v + t * RS + (((cg >> 1) ^ ((t >> 3) & 7)) << 4) + (cg & 1) * 8);
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) col[ch][e] = w[ch];
    }
    const int nv = ntok - t0;
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      T* dst = static_cast<T*>(a.vt) + head * a.vt_hs + (size_t)(cg * CH + ch) * a.vt_ld + tile0 + t0;
      if (nv >= TOK) {
        *reinterpret_cast<rowv*>(dst) = col[ch];
      } else {
#pragma unroll
        for (int e = 0; e < TOK; ++e)
          if (e < nv) dst[e] = col[ch][e];
      }
    }
  }
}

// One workgroup per (64-token tile, head).  K: each thread moves 16-byte chunks
// of a token's row, rotating pairs in fp32.  V: the tile goes into LDS as
// whole 16-byte chunks, then to V^T (store_vt).
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = D / VEC;                 // chunks per row
  constexpr int RS = D * (int)sizeof(T);       // LDS row stride (bytes)
  __shared__ __attribute__((aligned(16))) char s_v[64 * RS];
  const int tile0 = blockIdx.x * 64;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int ntok = min(64, a.T - tile0);
  const bool rot = a.k_rot && has_rope(a.rope);
  // every load first (RoPE table entries, then the K and V rows), then the
  // rotations and stores; rows past the block's end load its last row and
  // store nothing, so no load sits in a branch
  constexpr int IT = 64 * CPR / 256;
  static_assert(IT * 256 == 64 * CPR, "tile of 64 rows in whole passes of 256 threads");
  float2 cs[IT][VEC / 2];
  if (rot) {
    const RopeSel rs(a.rope);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
      int f, y, x;
      token_fyx(tile0 + r, a.rope.grid_h, a.rope.grid_w, f, y, x);
#pragma unroll
      for (int e = 0; e < VEC; e += 2) cs[it][e / 2] = rs.cs(c * VEC + e, a.t_row0 + f, y, x);
    }
  }
  typedef T chunk __attribute__((ext_vector_type(VEC)));   // one 16-byte chunk
  chunk kraw[IT], vraw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
    const size_t src = ((size_t)(tile0 + r) * a.H + head) * D + c * VEC;
    kraw[it] = *reinterpret_cast<const chunk*>(static_cast<const T*>(a.k_in) + src);
    vraw[it] = *reinterpret_cast<const chunk*>(static_cast<const T*>(a.v_in) + src);
  }
  // raw K rows (a context rotated per block, and the conv) as soon as they
  // arrive, V rows into LDS unguarded (rows past the end are never read
  // back), K rotated in registers, then the guarded rotated-K stores
  if (a.k_raw) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
      if (r < ntok)
        *reinterpret_cast<chunk*>(static_cast<T*>(a.k_raw) + head * a.k_raw_hs + (size_t)(tile0 + r) * D + c * VEC) =
            kraw[it];
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
    *reinterpret_cast<chunk*>(s_v + r * RS + ((c ^ ((r >> 3) & 7)) << 4)) = vraw[it];
  }
  chunk kout[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    kout[it] = kraw[it];
    if (rot) {
#pragma unroll
      for (int e = 0; e < VEC; e += 2) {
        float u0 = to_f(kraw[it][e]), u1 = to_f(kraw[it][e + 1]);
        rope_rot(u0, u1, cs[it][e / 2]);
        kout[it][e] = from_f<T>(u0);
        kout[it][e + 1] = from_f<T>(u1);
      }
    }
  }
  if (a.k_rot) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
      if (r < ntok)
        *reinterpret_cast<chunk*>(static_cast<T*>(a.k_rot) + head * a.k_rot_hs +
                                  (size_t)(a.k_rot_off + tile0 + r) * D + c * VEC) = kout[it];
    }
  }
  __syncthreads();
  store_vt<T, D>(a, s_v, tile0, head, ntok);
}

// OCP E4M3 ("fn": bias 7, 3 mantissa bits, largest finite 448).  Exponent of
// the power-of-two scale of a group whose largest magnitude is a: the
// smallest e with a * 2^-e <= 448 (0 for a = 0), clamped to [-120, 120], so
// values / 2^e never overflow E4M3 and the division is exact.
__device__ __forceinline__ int e4m3_exponent(float a) {
  if (!(a > 0.f)) return 0;
  int e = __builtin_amdgcn_frexp_expf(a) - 9;          // a * 2^-e in [256, 512)
  if (__builtin_amdgcn_ldexpf(a, -e) > 448.f) ++e;
  return min(120, max(-120, e));
}

// Four fp32 values (already divided by the scale) -> four E4M3 bytes, first
// value in the low byte; v_cvt_pk_fp8_f32 rounds to nearest, ties to even.
// The first convert writes the low half-word and keeps the high one from
// its third operand, which the second convert then overwrites: x0's own bits
// serve, so the result can take x0's register and none is cleared for it.
__device__ __forceinline__ int e4m3_pack4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __float_as_int(x0), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// E4M3 V^T rows of one (64-token tile, head) from the token-major bf16 V tile
// in LDS (16-byte chunk c of row r at c ^ ((r >> 3) & 7)), each value times
// inv (the tile's 2^-e): a task is 4 channels x 16 tokens, read as 8-byte
// slices (4 channels of one token) and written as one 16-byte run per
// channel.  Tokens past the block's end are written as 0, the value the pad
// columns hold from the workspace clear.
__device__ __forceinline__ void store_vt8(const AppendArgs& a, const char* s_v, int tile0, int head,
                                          int ntok, float inv) {
  constexpr int RS = 128 * 2;
  const int task = threadIdx.x;
  if (task >= 32 * 4) return;              // 32 channel groups x 4 token groups
  const int cg = task >> 2, tg = task & 3;
  const int t0 = tg * 16;
  if (t0 >= ntok) return;
  float col[4][16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int t = t0 + e;
    const bf16x4 w = *reinterpret_cast<const bf16x4*>(s_v + t * RS + (((cg >> 1) ^ ((t >> 3) & 7)) << 4) + (cg & 1) * 8);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) col[ch][e] = t < ntok ? (float)w[ch] * inv : 0.f;
  }
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    uint4 o;
    o.x = (unsigned)e4m3_pack4(col[ch][0], col[ch][1], col[ch][2], col[ch][3]);
    o.y = (unsigned)e4m3_pack4(col[ch][4], col[ch][5], col[ch][6], col[ch][7]);
    o.z = (unsigned)e4m3_pack4(col[ch][8], col[ch][9], col[ch][10], col[ch][11]);
    o.w = (unsigned)e4m3_pack4(col[ch][12], col[ch][13], col[ch][14], col[ch][15]);
    *reinterpret_cast<uint4*>(static_cast<char*>(a.v8) + head * a.v8_hs + (size_t)(4 * cg + ch) * a.v8_ld +
                              tile0 + t0) = o;
  }
}

// FP8 key cache append (bf16 inputs, D = 128): K rotated in fp32, then stored
// as E4M3 with one power-of-two scale per (64-token tile, head) -- the
// tile's largest |K~| reduced over the workgroup -- and the tile exponent
// written beside the rows.  V goes to V^T as in append_kernel (bf16, when
// vt is set) and, for the FP8 KV cache (v8 set), to E4M3 V^T with its own
// tile scale, the same rule over the tile's largest |V|.
__global__ __launch_bounds__(256) void append_k8_kernel(AppendArgs a) {
  constexpr int D = 128, VEC = 8, CPR = D / VEC, RS = D * 2, IT = 64 * CPR / 256;
  __shared__ __attribute__((aligned(16))) char s_v[64 * RS];
  __shared__ float s_max[4], s_vmax[4];
  const int tile0 = blockIdx.x * 64;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int ntok = min(64, a.T - tile0);
  const bool rope = has_rope(a.rope);
  // every load first (RoPE table entries, then the K and V rows); rows past
  // the block's end load its last row, count as 0 and store nothing
  float2 cs[IT][VEC / 2];
  if (rope) {
    const RopeSel rs(a.rope);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
      int f, y, x;
      token_fyx(tile0 + r, a.rope.grid_h, a.rope.grid_w, f, y, x);
#pragma unroll
      for (int e = 0; e < VEC; e += 2) cs[it][e / 2] = rs.cs(c * VEC + e, a.t_row0 + f, y, x);
    }
  }
  bf16x8 kraw[IT];
  uint4 vraw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
    const size_t src = ((size_t)(tile0 + r) * a.H + head) * D + c * VEC;
    kraw[it] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.k_in) + src);
    vraw[it] = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.v_in) + src);
  }
  // V rows into LDS unguarded (rows past the end are never read back), raw K
  // (a context rotated per block, and the conv) stored for live rows
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
    *reinterpret_cast<uint4*>(s_v + r * RS + ((c ^ ((r >> 3) & 7)) << 4)) = vraw[it];
  }
  if (a.k_raw) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
      if (r < ntok)
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.k_raw) + head * a.k_raw_hs + (size_t)(tile0 + r) * D +
                                   c * VEC) = kraw[it];
    }
  }
  float kr[IT][VEC];
  float amax = 0.f, vmax = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR;
    const bool live = r < ntok;
#pragma unroll
    for (int e = 0; e < VEC; ++e) kr[it][e] = live ? (float)kraw[it][e] : 0.f;
    if (rope) {
#pragma unroll
      for (int e = 0; e < VEC; e += 2) rope_rot(kr[it][e], kr[it][e + 1], cs[it][e / 2]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) amax = fmaxf(amax, fabsf(kr[it][e]));
    if (a.v8 && live) {
      const bf16x8 vv = *reinterpret_cast<const bf16x8*>(&vraw[it]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) vmax = fmaxf(vmax, fabsf((float)vv[e]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  }
  if ((tid & 63) == 0) {
    s_max[tid >> 6] = amax;
    s_vmax[tid >> 6] = vmax;
  }
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  vmax = fmaxf(fmaxf(s_vmax[0], s_vmax[1]), fmaxf(s_vmax[2], s_vmax[3]));
  const int ex = e4m3_exponent(amax);
  const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
    if (r >= ntok) continue;
    uint2 w;
    w.x = (unsigned)e4m3_pack4(kr[it][0] * inv, kr[it][1] * inv, kr[it][2] * inv, kr[it][3] * inv);
    w.y = (unsigned)e4m3_pack4(kr[it][4] * inv, kr[it][5] * inv, kr[it][6] * inv, kr[it][7] * inv);
    *reinterpret_cast<uint2*>(static_cast<char*>(a.k8) + head * a.k8_hs + (size_t)(tile0 + r) * D + c * VEC) = w;
  }
  if (tid == 0) a.kx[head * a.kx_hs + blockIdx.x] = ex;
  if (a.v8) {
    const int vex = e4m3_exponent(vmax);
    if (tid == 0) a.vx[head * a.vx_hs + blockIdx.x] = vex;
    store_vt8(a, s_v, tile0, head, ntok, __builtin_amdgcn_ldexpf(1.f, -vex));
  }
  if (a.vt) store_vt<__bf16, D>(a, s_v, tile0, head, ntok);
}

// ------------------------------------------------------------------ attention, bf16 MFMA
// Workgroup = 8 waves x 32 queries (BM = 256) of one head; key tiles of 64.
//
// Per wave and tile t: S(t) = K(t) Q^T (16 MFMA), softmax(t) (VALU: exp2,
// bf16 pack, fp32 row sum), PV(t) = V^T(t) P^T(t) (16 MFMA).  The waves form
// two groups of four (one wave of each group per SIMD) that run the same
// program half a tile apart: while group A issues its MFMA block [PV(t-1),
// S(t)] group B runs its softmax block, then they swap.  Whole-workgroup
// barriers between blocks keep the two groups in antiphase, so each SIMD's
// matrix core and vector ALU work at the same time.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16).  S^T: A = 32 keys x 16 channels
// (one 16-byte LDS read per lane), B = Q^T kept in registers.  MFMA row r is
// tile key pi(r) = 16*((r>>2)&1) + 4*(r>>3) + (r&3), so lane half h holds the
// 16 consecutive keys 16h..16h+15 of a 32-key block for query (lane & 31).
// O^T += V^T P^T reads A = V^T as 8 consecutive keys of one channel (one
// 16-byte LDS read) and B = P^T straight from registers: contraction index
// k = 8h + e stands for key 16h + 8*part + e on both operands.  A query's
// scores sit in lanes l and l^32.
//
// K/V tiles move HBM -> LDS with buffer_load ... lds (no register staging),
// three stages deep: tile t+2 is loaded (by group B, its 8 chunk loads per
// wave spread over its exponentials) while tiles t and t-1 are read.  LDS
// layouts are XOR-swizzled so that every 16-lane phase of a ds_read_b128
// touches all 64 banks once (gfx950 LDS: 64 banks x 4 B, 16 lanes per cycle).
// Loads are unpredicated: a partial tile reads the zeroed pad rows/columns
// of its buffer and its scores beyond the segment are masked to -inf.
// Softmax in log2 units with a lazily moved running max m: the S product
// starts from C = -m, so the accumulators hold s - m and P = exp2(S) needs
// no subtraction.  The first tile sets m to its exact row max.  Later tiles
// keep m unless a lane's partial row sum of P exceeds 2^8 (which any
// P > 2^8 forces); only then is the row max taken, m raised to it, O and l
// rescaled and P recomputed.  So P <= 2^8 always, and m never exceeds the
// true running max (l >= 1, no underflow).
constexpr int ABM = 256, ABN = 64, AD = 128, AWAVES = 8;
static_assert(ABM == kAttnBM, "unit rows");
constexpr int KT_BYTES = ABN * AD * 2;
constexpr int VT_BYTES = AD * ABN * 2;
constexpr int KT8_BYTES = ABN * AD;      // FP8 K tile: 64 rows x 128 bytes
constexpr int VT8_BYTES = AD * ABN;      // FP8 V^T tile: 128 channel rows x 64 bytes
constexpr int NSTAGE = 3;
constexpr float kSumLimit = 256.0f;     // lane partial row sum of P that forces a rescale
// FP8 V: P is packed as E4M3 at unit scale, so P <= 448 (E4M3's largest
// finite value) is the bound; log2(448) in the base-2 units of S.
constexpr float kLog2E4M3Max = 8.8073549f;
constexpr float kSumLimit8 = 448.0f;     // FP8 V: lane partial row sum of P that forces the row max test
constexpr float kHead8 = 3.0f;           // FP8 V: m = ceil(row max) - kHead8, largest P in (4, 8]
constexpr int kFragAhead = 3;            // LDS reads in flight ahead of the MFMA that uses them

// K tile: 64 rows x 16 chunks of 16 B.  Rows read together by a 16-lane phase
// are {0-7, 16-23} (+8, +32): (r & 7) | ((r & 16) >> 1) separates all 16.
__device__ __forceinline__ int kswz(int r) { return (r & 7) | ((r & 16) >> 1); }
// V^T tile: 128 rows x 8 chunks; two rows share a 256-B bank line.
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }
__device__ __forceinline__ int kperm(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }
// FP8 K tile: 64 rows x 8 chunks of 16 B (two rows per 256-B bank line).  A
// 16-lane phase reads one chunk from each of the rows {0-7, 16-23} (+8,
// +32); (r & 1) picks the bank half and this swizzle the chunk position, so
// the 16 reads cover the 64 banks once.
__device__ __forceinline__ int k8swz(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
// FP8 V^T tile: 128 channel rows x 4 chunks of 16 B (four rows per 256-B bank
// line).  A 16-lane phase reads the same logical chunk of 16 consecutive
// rows; rows r and r + 4 then sit at different chunk positions, so the 16
// reads cover the 64 banks once.
__device__ __forceinline__ int v8swz(int d) { return (d >> 2) & 3; }

__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs; give
  // each XCD a contiguous range of logical ids so one head's query tiles share
  // an L2.
  const int xcd = bid & 7, q = nwg >> 3, r = nwg & 7;
  return xcd * q + min(xcd, r) + (bid >> 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

// Workgroup barrier without a memory fence (tile loads are waited for
// explicitly with vmcnt before the barrier that publishes them).  The
// scheduling fences keep each block's instructions on its side.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + 2 GiB), stride 0 (base uniform).
__device__ __forceinline__ i32x4 buffer_rsrc(const char* base) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = (int)__builtin_amdgcn_readfirstlane((unsigned)b);
  r[1] = (int)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu);
  r[2] = 0x7fffffff;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from buffer (voff + soff) into LDS at lds_base + 16*lane
// (buffer_load_dwordx4 ... lds).  Written in asm so that the compiler does
// not treat every later LDS read as waiting on it: the caller waits with
// vmcnt(0) before the barrier that publishes the tile.  No register output.
// The LDS address goes in as an operand bound to m0 ("{m0}"), so the compiler
// writes m0 itself and knows it is live.
// The compiler's hazard checks do not look inside asm, so the asm provides
// the wait states a memory instruction needs itself: an SGPR written by a
// VALU instruction (v_readlane reloading a spilled SGPR, v_readfirstlane)
// may be read by a VMEM instruction only 5 wait states later, and the load
// reads the descriptor and the scalar offset from SGPRs (and m0, written by
// a scalar move, 1 wait state later).  s_nop 4 gives all 5 whatever
// precedes the asm.  With fewer, a build whose descriptor was reloaded from
// spill lanes just before a load read a stale descriptor and faulted.
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned voff, unsigned soff, unsigned lds_base) {
  // the scalar offset must sit in an SGPR, never a folded literal (the
  // descriptor and the LDS address come from registers anyway; marking them
  // as rewritten here would make the compiler copy them for every load)
  asm volatile("" : "+s"(soff));
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_base)
      : "memory");
}

// Two such loads from one descriptor, the second to LDS 4096 bytes on, in one
// asm block, so that they share its 5 wait states: m0 is an in/out operand
// (the block moves it to the second load's LDS address), and the second load
// reads it one wait state after that write.
__device__ __forceinline__ void dma16x2(i32x4 rsrc, unsigned voff0, unsigned soff0, unsigned voff1,
                                        unsigned soff1, unsigned lds_base) {
  asm volatile("" : "+s"(soff0), "+s"(soff1));
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %5 offen lds"
      : "+{m0}"(lds_base)
      : "v"(voff0), "v"(voff1), "s"(rsrc), "s"(soff0), "s"(soff1)
      : "memory", "scc");
}

// Tile cursor over the context segments: every full 64-key tile of every
// segment first (phase 0), then the partial tail tile of each segment whose
// length is not a multiple of 64 (phase 1).  Attention does not depend on
// key order.  All fields are wave-uniform.
struct TileCursor {
  int phase, sg, j0, n;   // n: length of segment sg (0 past the end)
  int lim;                // n in phase 0, else 0: the next tile is j0 + 64 of the
                          // same segment when j0 + 128 <= lim (the common case)
};

template <bool SPLIT, bool KF8, bool VF8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  static_assert(KF8 || !VF8, "the FP8 V cache comes with the FP8 key cache");
  constexpr int KTB = KF8 ? KT8_BYTES : KT_BYTES;   // K tile bytes in LDS
  constexpr int VTB = VF8 ? VT8_BYTES : VT_BYTES;   // V^T tile bytes in LDS
  constexpr int SB = KTB + VTB;                       // stage bytes
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * SB];
  __shared__ const char* s_k[kMaxSeg];      // segment K / V^T of the current head
  __shared__ const char* s_v[kMaxSeg];
  __shared__ const char* s_kb[kMaxSeg];     // head 0, with per-head strides
  __shared__ const char* s_vb[kMaxSeg];
  __shared__ long long s_khs[kMaxSeg];
  __shared__ long long s_vhs[kMaxSeg];
  __shared__ int s_n[kMaxSeg];
  __shared__ int s_ld[kMaxSeg];
  __shared__ const int* s_x[kMaxSeg];       // FP8 K: tile exponents of the current head
  __shared__ const int* s_xb[kMaxSeg];
  __shared__ long long s_xhs[kMaxSeg];
  __shared__ const int* s_vx[kMaxSeg];      // FP8 V: tile exponents of the current head
  __shared__ const int* s_vxb[kMaxSeg];
  __shared__ long long s_vxhs[kMaxSeg];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform by construction
  const int group = wave >> 2, gw = wave & 3;           // ping-pong group, wave in group
  const int hh = lane >> 5, col = lane & 31;
  const int nqt = (a.T + ABM - 1) / ABM;
  const int nseg = __builtin_amdgcn_readfirstlane(a.nseg);

  // segment table into LDS; one segment per wave, compile-time indices into
  // the argument block (a run-time index would copy it to scratch memory)
#pragma unroll
  for (int g = 0; g < kMaxSeg; g += AWAVES) {
    const int gg = g + wave;
    if (gg < nseg && lane == 0) {
      Seg sg;
#pragma unroll
      for (int w = 0; w < AWAVES; ++w)
        if (g + w < kMaxSeg && w == wave) sg = a.seg[g + w];
      const char* kb;
      const char* vb;
      long long khs, vhs;
      int ld;
      if (sg.dyn >= 0) {
        const int slot = a.sel_slots[sg.dyn];
        kb = a.slot_base + (long long)slot * a.slot_bytes;
        vb = kb + a.slot_v_off;
        khs = a.slot_k_hs;
        vhs = a.slot_v_hs;
        ld = a.slot_v_ld;
        if constexpr (KF8) {
          s_xb[gg] = reinterpret_cast<const int*>(kb + a.slot_kx_off);
          s_xhs[gg] = a.slot_kx_hs;
        }
        if constexpr (VF8) {
          s_vxb[gg] = reinterpret_cast<const int*>(kb + a.slot_vx_off);
          s_vxhs[gg] = a.slot_vx_hs;
        }
        if (sg.k) {                      // K rotated into the context-K buffer
          kb = static_cast<const char*>(sg.k);
          khs = sg.k_hs;
          if constexpr (KF8) {
            s_xb[gg] = sg.kx;
            s_xhs[gg] = sg.kx_hs;
          }
        }
      } else {
        kb = static_cast<const char*>(sg.k);
        vb = static_cast<const char*>(sg.v);
        khs = sg.k_hs;
        vhs = sg.v_hs;
        ld = sg.v_ld;
        if constexpr (KF8) {
          s_xb[gg] = sg.kx;
          s_xhs[gg] = sg.kx_hs;
        }
        if constexpr (VF8) {
          s_vxb[gg] = sg.vx;
          s_vxhs[gg] = sg.vx_hs;
        }
      }
      s_kb[gg] = kb;
      s_vb[gg] = vb;
      s_khs[gg] = khs;
      s_vhs[gg] = vhs;
      s_n[gg] = sg.n;
      s_ld[gg] = ld;
    }
  }

  // Q of a unit: lane holds Q~[q][16s + 8h .. +7] for s = 0..7, rotated,
  // scaled by softmax_scale*log2(e), rounded to bf16.
  bf16x8 qreg[8];
  // FP8 K: the same Q~ as E4M3 with one power-of-two scale per query, lane
  // holding channels 64 s2 + 32 h .. +31 (s2 = 0, 1) as 32 bytes; qsc is the
  // query's scale as an E8M0 exponent (127 + e).
  i32x8 qreg8[2];
  int qsc = 127;
  __syncthreads();

  // ---- tile enumeration (segment metadata read as wave-uniform values)
  auto seg_n = [&](int g) { return __builtin_amdgcn_readfirstlane(s_n[g]); };
  auto first_tail = [&](int from) {
    int g = from;
    while (g < nseg && (seg_n(g) & (ABN - 1)) == 0) ++g;
    return g;
  };
  auto first_full = [&](int from) {
    int g = from;
    while (g < nseg && seg_n(g) < ABN) ++g;
    return g;
  };
  // cursor at tile k of the enumeration (full tiles of each segment in
  // order, then the partial tails)
  auto cursor_find = [&](int k) {
    TileCursor c{0, nseg, 0, 0, 0};
    for (int g = 0; g < nseg; ++g) {
      const int f = seg_n(g) / ABN;
      if (k < f) {
        c.sg = g;
        c.j0 = k * ABN;
        c.n = seg_n(g);
        return c;
      }
      k -= f;
    }
    c.phase = 1;
    for (int g = 0; g < nseg; ++g) {
      if (seg_n(g) & (ABN - 1)) {
        if (k == 0) {
          c.sg = g;
          c.n = seg_n(g);
          c.j0 = c.n & ~(ABN - 1);
          return c;
        }
        --k;
      }
    }
    return c;
  };
  // (the fields are re-read as wave-uniform: the cursor is carried across
  // the piece loop, where the compiler no longer proves it uniform)
  auto cursor_seek = [&](int k) {
    TileCursor c = cursor_find(__builtin_amdgcn_readfirstlane(k));
    c.phase = __builtin_amdgcn_readfirstlane(c.phase);
    c.sg = __builtin_amdgcn_readfirstlane(c.sg);
    c.j0 = __builtin_amdgcn_readfirstlane(c.j0);
    c.n = __builtin_amdgcn_readfirstlane(c.n);
    c.lim = (c.phase == 0 && c.sg < nseg) ? c.n : 0;
    return c;
  };
  // The next tile of a cursor.  The common case (the next full tile of the
  // same segment) is one compare that falls through; segment changes take
  // the out-of-line path.
  auto advance_slow = [&](TileCursor& c) {
    if (c.sg < nseg) {
      if (c.phase == 0) {
        c.j0 += ABN;
        if (c.j0 + ABN > c.n) {
          c.sg = first_full(c.sg + 1);
          c.j0 = 0;
          if (c.sg >= nseg) {
            c.phase = 1;
            c.sg = first_tail(0);
          }
          if (c.sg < nseg) {               // else past the unit's last tile (load cursor only)
            c.n = seg_n(c.sg);
            c.j0 = c.phase == 1 ? c.n & ~(ABN - 1) : 0;
          }
        }
      } else {
        c.sg = first_tail(c.sg + 1);
        if (c.sg < nseg) {
          c.n = seg_n(c.sg);
          c.j0 = c.n & ~(ABN - 1);
        }
      }
    }
    c.lim = (c.phase == 0 && c.sg < nseg) ? c.n : 0;
  };
  auto advance = [&](TileCursor& c) {
    const int nj = c.j0 + ABN;
    if (__builtin_expect(nj + ABN <= c.lim, 1)) {
      c.j0 = nj;
      return;
    }
    advance_slow(c);
  };
  int NT = 0;
  for (int g = 0; g < nseg; ++g) NT += (seg_n(g) + ABN - 1) / ABN;
  // split launch: the units from unit0 on (fewer than a round; the full
  // rounds ran in a plain launch before it), each cut into rP key-tile parts
  // (part p = tiles [NT p / rP, NT (p+1) / rP))
  // (rP is set by the host, 1 <= rP <= NT, rP * rU <= kStreamWG)
  const int rU = SPLIT ? a.H * nqt - a.unit0 : 0;
  const int rP = SPLIT ? a.parts : 1;

  // ---- tile loads: chunk p = (4i + w)*64 + lane of a tile lands at LDS p*16
  // (w = wave within the loading group of four); the tile's first key enters
  // as the scalar offset of the buffer load.
  int cur_sg = -1, cur_ld = 0;
  i32x4 krs = {0, 0, 0, 0}, vrs = {0, 0, 0, 0};
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_ptr_t)lds;
  // A tile's load = scalar set-up (segment descriptors, LDS and key offsets)
  // then 8 chunk loads (4 of K, 4 of V) that the softmax interleaves with its
  // exponentials: the CU's address unit takes each 1 KB chunk in ~16 cycles,
  // so issuing all 32 of a tile back to back would stall the loading waves.
  unsigned ld_kt = 0, ld_j0 = 0;
  // Per-lane chunk offsets.  Chunk i of a K tile sits at vk[i & 1] + (i >> 1)
  // * 8192 and chunk i of a V^T tile at vv + i * 32 rows: every i-dependent
  // part is uniform and goes into the scalar offset, so three registers
  // serve all eight loads (vv changes with the segment's row stride).
  auto k_off = [&](int i) {
    const int p = (4 * i + gw) * 64 + lane;
    return (unsigned)((p >> 4) * 256 + (((p & 15) ^ kswz(p >> 4)) << 4));
  };
  const unsigned vk0 = k_off(0), vk1 = k_off(1);
  // FP8 K (64 rows of 128 B): chunk p = (4i + w)*64 + lane of a tile holds row
  // p >> 3 = 32i + 8w + (lane >> 3), chunk (p & 7) ^ k8swz(row); that swizzle
  // does not depend on i, so one register serves both loads (+4096 i).
  const unsigned vk8 = (unsigned)(gw * 1024 + (lane >> 3) * 128 +
                                  (((lane & 7) ^ (((lane >> 4) & 3) | (((gw >> 1) & 1) << 2))) << 4));
  // FP8 V^T (128 rows of 64 B): chunk p = (4i + w)*64 + lane of a tile holds
  // row p >> 2 = 64i + 16w + (lane >> 2), chunk (p & 3) ^ v8swz(row); the
  // swizzle is (lane >> 4) & 3 for every i, so one register serves both loads
  // (+ 64 rows per i in the scalar offset).
  unsigned vv = 0;
  auto issue_setup = [&](const TileCursor& c, int stage) {
    if (c.sg != cur_sg) {
      cur_sg = c.sg;
      krs = buffer_rsrc(uniform_ptr(s_k[c.sg]));
      vrs = buffer_rsrc(uniform_ptr(s_v[c.sg]));
      cur_ld = __builtin_amdgcn_readfirstlane(s_ld[c.sg]);
      if constexpr (VF8) {
        vv = (unsigned)((gw * 16 + (lane >> 2)) * cur_ld + (((lane & 3) ^ ((lane >> 4) & 3)) << 4));
      } else {
        const int p = gw * 64 + lane;
        vv = (unsigned)((p >> 3) * cur_ld * 2 + (((p & 7) ^ vswz(p >> 3)) << 4));
      }
    }
    ld_kt = __builtin_amdgcn_readfirstlane(lds0 + stage * SB + gw * 1024);
    ld_j0 = __builtin_amdgcn_readfirstlane((unsigned)c.j0);
  };
  auto uni4 = [](i32x4 r) {
    i32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (int)__builtin_amdgcn_readfirstlane((unsigned)r[e]);
    return u;
  };
  // bf16 K: k = 0..3 K chunks, 4..7 V chunks.  FP8 K: 0..1 K, 2..5 V, 6..7
  // none.  FP8 K and V: 0..1 K, 2..3 V, 4..7 none.
  constexpr int NCHUNK = VF8 ? 4 : (KF8 ? 6 : 8);
  // FP8 K and V: chunks k and k + 1 go in together at even k (their LDS
  // places are 4096 bytes apart), so the pair shares one set of wait states
  // (measured faster there; on the other paths single loads were faster)
  auto issue_chunk = [&](int k) {
    const unsigned j0 = __builtin_amdgcn_readfirstlane(ld_j0);
    const unsigned kt = __builtin_amdgcn_readfirstlane(ld_kt);
    const unsigned ld = __builtin_amdgcn_readfirstlane((unsigned)cur_ld);
    if constexpr (VF8) {
      if (k == 0)
        dma16x2(uni4(krs), vk8, j0 * 128u, vk8, j0 * 128u + 4096u, kt);
      else if (k == 2)
        dma16x2(uni4(vrs), vv, j0, vv, j0 + 64u * ld, kt + KTB);
    } else if constexpr (KF8) {
      if (k < 2)
        dma16(uni4(krs), vk8, j0 * 128u + (unsigned)k * 4096u, kt + k * 4096);
      else if (k < 6)
        dma16(uni4(vrs), vv, j0 * 2u + (unsigned)(k - 2) * 64u * ld, kt + KTB + (k - 2) * 4096);
    } else {
      const int i = k & 3;
      if (k < 4)
        dma16(uni4(krs), (i & 1) ? vk1 : vk0, j0 * 256u + (unsigned)(i >> 1) * 8192u, kt + i * 4096);
      else
        dma16(uni4(vrs), vv, j0 * 2u + (unsigned)i * 64u * ld, kt + KTB + i * 4096);
    }
  };
  auto issue = [&](const TileCursor& c, int stage) {   // by one group of four waves
    issue_setup(c, stage);
#pragma unroll
    for (int k = 0; k < NCHUNK; ++k) issue_chunk(k);
  };

  // ---- per-wave state
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  // m_run: running row max (log2 units); negm = -m_run in every element, the
  // C operand of the S product.  Both are set by the first tile.
  float m_run = 0.f, l_run = 0.f;
  f32x16 negm = f32x16{};
  f32x16 sacc[2];
  bf16x8 pb[2][2];
  // FP8 V: P^T as the B operand of the scaled 32x32x64 MFMA, E4M3 at unit
  // scale.  Lane half h holds, as contraction indices 32h .. 32h+31, the
  // keys 16h .. 16h+15 (sacc[0]) then 32+16h .. 32+16h+15 (sacc[1]): the
  // lane's own scores in register order, so no exchange between lanes.
  i32x8 pb8;
  i32x8 kf[4];                             // FP8 K fragments of the S product

  // MFMA block: PV of one tile (16 MFMA, V^T fragments) then, optionally, S of
  // the next (16 MFMA, K fragments).  Fragments rotate through 4 registers
  // sets with LDS reads issued 3 MFMAs ahead, so the matrix core does not
  // wait on LDS latency; consecutive MFMAs target different accumulators.
  // fragment registers of the MFMA block; the first kFragAhead are read by
  // m_prefetch before the barrier that opens the block (its V tile was
  // published a period earlier), so the block starts without LDS latency
  constexpr int AHEAD = kFragAhead;
  bf16x8 fr[AHEAD + 1];
  auto pv_frag = [&](const char* vt, int i) -> bf16x8 {   // PV step: (mb, part, db), db fastest
    const int mb = i >> 3, part = (i >> 2) & 1, db = i & 3;
    const int d = 32 * db + col, c = 4 * mb + 2 * hh + part;
    return *reinterpret_cast<const bf16x8*>(vt + d * 128 + ((c ^ vswz(d)) << 4));
  };
  auto m_prefetch = [&](const char* vt) {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) fr[i] = pv_frag(vt, i);
  };
  auto m_block = [&](const char* vt, const char* kt, auto with_s) {
    constexpr int NSTEP = decltype(with_s)::value ? 32 : 16;
    const int r0 = kperm(col), r1 = 32 + kperm(col);
    auto frag = [&](int i) -> bf16x8 {
      if (i < 16) return pv_frag(vt, i);
      const int j = i - 16, st = j >> 1, r = (j & 1) ? r1 : r0;   // S step: (s, key block)
      const int c = 2 * st + hh;
      return *reinterpret_cast<const bf16x8*>(kt + r * 256 + ((c ^ kswz(r)) << 4));
    };
    auto step = [&](int i, const bf16x8& f) {
      if (i < 16) {
        const int mb = i >> 3, part = (i >> 2) & 1, db = i & 3;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pb[mb][part], o[db], 0, 0, 0);
      } else {
        const int j = i - 16, st = j >> 1, blk = j & 1;
        sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qreg[st], st ? sacc[blk] : negm, 0, 0, 0);
      }
    };
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + AHEAD < NSTEP) fr[(i + AHEAD) % (AHEAD + 1)] = frag(i + AHEAD);
      step(i, fr[i % (AHEAD + 1)]);
    }
    // instruction order: (read, MFMA) pairs, then the last MFMAs
#pragma unroll
    for (int i = 0; i < NSTEP - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  };
  auto s_only = [&](const char* kt) {    // S of the first tile (no PV yet)
    const int r0 = kperm(col), r1 = 32 + kperm(col);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int c = 2 * st + hh;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kt + r0 * 256 + ((c ^ kswz(r0)) << 4));
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kt + r1 * 256 + ((c ^ kswz(r1)) << 4));
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[st], st ? sacc[0] : f32x16{}, 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[st], st ? sacc[1] : f32x16{}, 0, 0, 0);
    }
  };
  // FP8 K: S^T = K Q^T as 4 scaled MFMAs (32x32x64, E4M3 x E4M3) per tile.
  // Fragment j = 2 s2 + blk: A = 32 keys (MFMA row r = tile row kperm(r) +
  // 32 blk) x channels 64 s2 .. +63, lane (col, h) holding channels
  // 64 s2 + 32 h .. +31 of its row (two 16-byte chunks); B = qreg8[s2].  The
  // A scale is the tile's exponent (uniform), the B scale the query's, so
  // the product is the dequantised one.  Row and lane layout of the result
  // are those of the bf16 product.
  auto k8_frag = [&](const char* kt, int j) -> i32x8 {
    const int r = 32 * (j & 1) + kperm(col);
    const int p = (4 * (j >> 1) + 2 * hh) ^ k8swz(r);
    const i32x4 lo = *reinterpret_cast<const i32x4*>(kt + r * 128 + (p << 4));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(kt + r * 128 + ((p ^ 1) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto s8_step = [&](int j, int sa, const f32x16& c0) {
    const int blk = j & 1, s2 = j >> 1;
    sacc[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[j], qreg8[s2], s2 ? sacc[blk] : c0,
                                                               0, 0, 0, sa, 0, qsc);
  };
  // first tile (no PV yet); sa = 127 + the tile's exponent
  auto s_only8 = [&](const char* kt, int sa) {
#pragma unroll
    for (int j = 0; j < 4; ++j) kf[j] = k8_frag(kt, j);
#pragma unroll
    for (int j = 0; j < 4; ++j) s8_step(j, sa, f32x16{});
  };
  // MFMA block of the FP8 path: PV (16 MFMA, V^T fragments 3 ahead as in
  // m_block) then S (4 scaled MFMA).  The K tile is read only inside the
  // block: it is published by the barrier that opens the block (the loading
  // group waits for its chunks before that barrier), unlike the V^T tile,
  // which m_prefetch may read earlier.  The eight K chunk reads follow the
  // PV reads from step 10 on (two reads at steps 10-12, two more with the
  // first scaled MFMA, which takes twice as long as a PV MFMA).
  auto m_block8 = [&](const char* vt, const char* kt, int sa) {
    static_assert(AHEAD == 3, "read slots below assume 3 reads ahead");
    i32x4 h[8];                          // chunk 2j + half of fragment j
    auto k8_half = [&](int c) {
      const int j = c >> 1, r = 32 * (j & 1) + kperm(col);
      const int p = ((4 * (j >> 1) + 2 * hh) ^ k8swz(r)) ^ (c & 1);
      return *reinterpret_cast<const i32x4*>(kt + r * 128 + (p << 4));
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + AHEAD < 16) fr[(i + AHEAD) % (AHEAD + 1)] = pv_frag(vt, i + AHEAD);
      if (i >= 10) h[i - 10] = k8_half(i - 10);
      const int mb = i >> 3, part = (i >> 2) & 1, db = i & 3;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (AHEAD + 1)], pb[mb][part], o[db], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) kf[j] = __builtin_shufflevector(h[2 * j], h[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    h[6] = k8_half(6);
    h[7] = k8_half(7);
    kf[3] = __builtin_shufflevector(h[6], h[7], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < 4; ++j) s8_step(j, sa, negm);
    // instruction order: (read, MFMA) pairs up to step 9, (2 reads, MFMA)
    // for steps 10-12, (read, MFMA) for 13-15, then (2 reads, MFMA) and the
    // last three MFMAs
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int i = 10; i < 13; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int i = 13; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // MFMA block of the FP8 K and V path: PV as 4 scaled MFMAs (32x32x64, A =
  // the E4M3 V^T fragment of channel block db, B = pb8, A scale the V tile's
  // exponent, B scale 2^0), then S as 4 scaled MFMAs.  The V^T fragment of
  // channel row d = 32 db + col is its logical chunks h (keys 16h..16h+15)
  // and 2+h (keys 32+16h..); those of db = 0 are read by m_prefetch88 before
  // the barrier (the V tile was published a period earlier), the rest two
  // MFMAs ahead inside the block, with the K tile's reads after the barrier.
  i32x4 hv[8];
  auto v8_half = [&](const char* vt, int c) -> i32x4 {   // c = 2 db + which
    const int d = 32 * (c >> 1) + col;
    const int lc = (c & 1) ? 2 + hh : hh;
    return *reinterpret_cast<const i32x4*>(vt + d * 64 + ((lc ^ v8swz(d)) << 4));
  };
  auto m_prefetch88 = [&](const char* vt) {
    hv[0] = v8_half(vt, 0);
    hv[1] = v8_half(vt, 1);
  };
  auto m_block88 = [&](const char* vt, const char* kt, int sk, int sv, auto with_s_t) {
    constexpr bool with_s = decltype(with_s_t)::value;
    i32x4 hk[8];
    auto k8_half = [&](int c) {
      const int j = c >> 1, r = 32 * (j & 1) + kperm(col);
      const int p = ((4 * (j >> 1) + 2 * hh) ^ k8swz(r)) ^ (c & 1);
      return *reinterpret_cast<const i32x4*>(kt + r * 128 + (p << 4));
    };
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x8 vf = __builtin_shufflevector(hv[2 * db], hv[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pb8, o[db], 0, 0, 0, sv, 0, 127);
      if (db < 3) {
        hv[2 * db + 2] = v8_half(vt, 2 * db + 2);
        hv[2 * db + 3] = v8_half(vt, 2 * db + 3);
      }
      if (with_s) {
        hk[2 * db] = k8_half(2 * db);
        hk[2 * db + 1] = k8_half(2 * db + 1);
      }
    }
    if (with_s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) kf[j] = __builtin_shufflevector(hk[2 * j], hk[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int j = 0; j < 4; ++j) s8_step(j, sk, negm);
    }
    // instruction order: (MFMA, then the next fragments' reads) four times,
    // then the S MFMAs
    constexpr int NR = with_s ? 4 : 2;      // reads after each of the first three MFMAs
#pragma unroll
    for (int db = 0; db < 3; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (with_s) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };
  // E8M0 A scale (127 + exponent) of the FP8 K tile at cursor c, read through
  // the scalar cache: the exponents were written by an earlier launch.
  // The segment's exponent pointer is re-read from LDS only when the segment
  // changes (x_sg is reset with each piece's table).
  int x_sg = -1;
  const char* x_ptr = nullptr;
  auto tile_scale = [&](const TileCursor& c) -> int {
    typedef const __attribute__((address_space(4))) int* const_int_ptr;
    if (__builtin_expect(c.sg != x_sg, 0)) {
      x_sg = c.sg;
      x_ptr = uniform_ptr(s_x[c.sg]);
    }
    return 127 + reinterpret_cast<const_int_ptr>(reinterpret_cast<uintptr_t>(x_ptr))[c.j0 >> 6];
  };
  // the same for the FP8 V tile at cursor c
  int vx_sg = -1;
  const char* vx_ptr = nullptr;
  auto vtile_scale = [&](const TileCursor& c) -> int {
    typedef const __attribute__((address_space(4))) int* const_int_ptr;
    if (__builtin_expect(c.sg != vx_sg, 0)) {
      vx_sg = c.sg;
      vx_ptr = uniform_ptr(s_vx[c.sg]);
    }
    return 127 + reinterpret_cast<const_int_ptr>(reinterpret_cast<uintptr_t>(vx_ptr))[c.j0 >> 6];
  };
  auto mask_tail = [&](int nvalid) {
    if (nvalid < ABN) {
      asm volatile("" ::: "memory");     // keep the tail mask a real branch
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * mb + 16 * hh + i >= nvalid) sacc[mb][i] = -INFINITY;
    }
  };
  // row max of the tile's S: four max3 chains over the lane's 32 scores, then
  // lanes l and l^32 (same query) exchange
  auto lane_max = [&]() {                 // over this lane's 32 keys of its row
    float c4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& v = sacc[q >> 1];
      const int b = (q & 1) * 8;
      float x = __builtin_fmaxf(__builtin_fmaxf(v[b], v[b + 1]), v[b + 2]);
      x = __builtin_fmaxf(__builtin_fmaxf(x, v[b + 3]), v[b + 4]);
      x = __builtin_fmaxf(__builtin_fmaxf(x, v[b + 5]), v[b + 6]);
      c4[q] = __builtin_fmaxf(x, v[b + 7]);
    }
    return __builtin_fmaxf(__builtin_fmaxf(c4[0], c4[1]), __builtin_fmaxf(c4[2], c4[3]));
  };
  auto row_max = [&]() {                  // lanes l and l ^ 32 hold a row's 64 keys
    const float mx = lane_max();
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // P = exp2(S - shift) packed to bf16; returns the lane's partial row sum of
  // P in fp32 (four chains of plain adds: the bf16 dot instructions would
  // share the matrix core with the other group's MFMAs)
  // (FP8 V: P packed to E4M3 at unit scale, four values per word; the
  // running max keeps every P within E4M3's largest finite value, 448)
  auto exp_pack = [&](float shift, auto shifted, auto&& hook) {
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float e4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * g + u;
          const float x = decltype(shifted)::value ? sacc[mb][i] - shift : sacc[mb][i];
          const float e = __builtin_amdgcn_exp2f(x);
          e4[u] = e;
          if constexpr (!VF8) pb[mb][i >> 3][i & 7] = (__bf16)e;
          // a chain's first term is stored, not added to 0 (the same value:
          // exp2 is never -0), which saves four adds per tile
          if ((g & 1) == 0 && u == 0) ls[2 * mb + (g >> 1)] = e;
          else ls[2 * mb + (g >> 1)] += e;
        }
        if constexpr (VF8) pb8[4 * mb + g] = e4m3_pack4(e4[0], e4[1], e4[2], e4[3]);
        hook(4 * mb + g);
      }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto no_hook = [](int) {};
  auto set_m = [&](float m) {
    m_run = m;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m;
  };
  // first tile: S holds raw scores; m = the exact row max.  FP8 V: m moves
  // only by whole numbers, starting at ceil(row max) - 3, so P = 2^(s - m)
  // is the row's P times a power of two, its largest value in (4, 8], and
  // its E4M3 codes are those of P under the row's own power-of-two scale
  // (E4M3's rounding is the same at every power of two, up to values in
  // its subnormal range, 2^9 below the largest); every rescale factor is
  // then an exact power of two.
  auto softmax_first = [&](int nvalid, auto&& load_hook) {
    mask_tail(nvalid);
    const float mx = row_max();
    const float m0 = VF8 ? ceilf(mx) - kHead8 : mx;
    set_m(m0);
    l_run = exp_pack(m0, std::true_type{}, load_hook);
  };
  // later tiles: S holds s - m
  auto softmax = [&](int nvalid, auto&& load_hook) {
    mask_tail(nvalid);
    float part = exp_pack(0.f, std::false_type{}, load_hook);
    if constexpr (VF8) {
      // a lane sum within 448 keeps each P within it; otherwise the row max
      // decides, and a row with a P above 448 moves m up by the whole number
      // that brings its largest P back into (4, 8].  With every P at most 8
      // until a row's max grows, a lane's 32 P sum to at most 256 (a flat
      // row, as the zeroed rows past a block's end are, included), so the
      // test fires only around a grown max.
      if (__any(!(part <= kSumLimit8))) {
        const float rm = row_max();
        const float d = rm > kLog2E4M3Max ? ceilf(rm - kHead8) : 0.f;   // 0: the row keeps m
        const float alpha = __builtin_amdgcn_exp2f(-d);
        set_m(m_run + d);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        part = exp_pack(d, std::true_type{}, no_hook);
      }
    } else if (__any(!(part <= kSumLimit))) {
      const float d = fmaxf(row_max(), 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-d);
      set_m(m_run + d);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      part = exp_pack(d, std::true_type{}, no_hook);
    }
    l_run += part;
  };
  auto stage_of = [](int t) { return t % NSTAGE; };
  TileCursor xc{}, lc{};                   // next softmax tile, next load tile

  // final output of a unit's 256 rows: O / l in bf16
  auto write_out = [&](int head, int qrow) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qrow < a.T) {
      __bf16* op = static_cast<__bf16*>(a.out) + ((size_t)qrow * a.H + head) * AD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * j + e] * inv);
          *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hh) = w;
        }
    }
  };

  // ---- one piece: key tiles [ka, kb) of unit u = head * nqt + qt (NT tiles
  // per unit).  A piece of a cut unit (split launch only) is part j of
  // remainder unit v.
  auto piece = [&](int u, int ka, int kb, int v, int j) __attribute__((always_inline)) {
    const int head = __builtin_amdgcn_readfirstlane(u / nqt);
    const int qt = u - head * nqt;
    const int qrow = qt * ABM + wave * 32 + col;
    const int NP = kb - ka;                // key tiles of this piece, >= 1

    __syncthreads();                       // the previous piece is done with LDS
    if (tid < nseg) {
      s_k[tid] = s_kb[tid] + (KF8 ? 1 : 2) * head * s_khs[tid];
      s_v[tid] = s_vb[tid] + (VF8 ? 1 : 2) * head * s_vhs[tid];
      if constexpr (KF8) s_x[tid] = s_xb[tid] + head * s_xhs[tid];
      if constexpr (VF8) s_vx[tid] = s_vxb[tid] + head * s_vxhs[tid];
    }
    // Q of the unit: the RoPE table entries and the 8 row chunks of a lane
    // are loaded before the first use (rows past the block's end load its
    // last row and are zeroed)
    const bool valid = qrow < a.T;
    const int qr = valid ? qrow : a.T - 1;
    const bool rope = has_rope(a.rope);
    const __bf16* qp = static_cast<const __bf16*>(a.q) + ((size_t)qr * a.H + head) * AD;
    if constexpr (KF8) {   // Q of the unit as E4M3, one scale per query
      float2 cs[8][4];
      if (rope) {
        int f, y, x;
        token_fyx(qr, a.rope.grid_h, a.rope.grid_w, f, y, x);
        const RopeSel rsel(a.rope);
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            cs[k][e / 2] = rsel.cs(64 * (k >> 2) + 32 * hh + 8 * (k & 3) + e, a.t_row0 + f, y, x);
      }
      bf16x8 raw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) raw[k] = *reinterpret_cast<const bf16x8*>(qp + 64 * (k >> 2) + 32 * hh + 8 * (k & 3));
      float u[2][32];
      float mx = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int k = 4 * s2 + c4;
          float* w = &u[s2][8 * c4];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = valid ? (float)raw[k][e] : 0.f;
          if (rope) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) rope_rot(w[e], w[e + 1], cs[k][e / 2]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            w[e] *= a.qscale;
            mx = fmaxf(mx, fabsf(w[e]));
          }
        }
      // the query's other 64 channels sit in lane l ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const int eq = e4m3_exponent(mx);
      const float inv = __builtin_amdgcn_ldexpf(1.f, -eq);
      qsc = 127 + eq;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int w = 0; w < 8; ++w)
          qreg8[s2][w] = e4m3_pack4(u[s2][4 * w] * inv, u[s2][4 * w + 1] * inv, u[s2][4 * w + 2] * inv,
                                    u[s2][4 * w + 3] * inv);
    } else {
      float2 cs[8][4];
      if (rope) {
        int f, y, x;
        token_fyx(qr, a.rope.grid_h, a.rope.grid_w, f, y, x);
        const RopeSel rsel(a.rope);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int e = 0; e < 8; e += 2) cs[s][e / 2] = rsel.cs(16 * s + 8 * hh + e, a.t_row0 + f, y, x);
      }
      bf16x8 raw[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * hh);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = valid ? (float)raw[s][e] : 0.f;
        if (rope) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) rope_rot(u[e], u[e + 1], cs[s][e / 2]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[s][e] = (__bf16)(u[e] * a.qscale);
      }
    }
    __syncthreads();
    cur_sg = -1;
    x_sg = -1;
    vx_sg = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};
    m_run = 0.f;
    l_run = 0.f;
    negm = f32x16{};

    // ---- prologue: tiles 0 and 1 of the piece loaded by group 0 (all waves wait)
    xc = cursor_seek(ka);
    lc = xc;
    if (group == 0) {
      issue(lc, 0);
      advance(lc);
      if (NP > 1) issue(lc, 1);
    } else {
      advance(lc);
    }
    advance(lc);                           // lc -> tile 2
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

      if (NP > 0) {
        if (group == 1) wg_barrier();          // group B runs half a tile behind
        // M(0) = S(0)
        if constexpr (KF8) s_only8(lds + stage_of(0) * SB, tile_scale(xc));
        else s_only(lds + stage_of(0) * SB);
        wg_barrier();
        // Full periods: X(t) then M(t+1) = [PV(t), S(t+1)].  The first period
        // (exact max), the last loading period and the last tile are peeled, and
        // each group runs its own copy of the loop, so the steady loop body holds
        // a single softmax and MFMA-block variant and group B's chunk loads are
        // unconditional (pinned between the exponentials).
        // load: 0 = none, 1 = group B loads tile t+2
        auto period = [&](int t, auto first, auto load) {
          constexpr int LOAD = decltype(load)::value;
          if (LOAD == 1) issue_setup(lc, stage_of(t + 2));
          advance(lc);
          auto hook = [&](int k) {
            if constexpr (LOAD == 1) {
              __builtin_amdgcn_sched_barrier(0);
              issue_chunk(k);
              __builtin_amdgcn_sched_barrier(0);
            }
          };
          if constexpr (VF8) {
            // V scale of tile t (at the cursor, before it moves) and K scale
            // of tile t+1, read before the softmax so that their scalar
            // loads have returned by the MFMA block
            const int nvalid = xc.n - xc.j0;
            const int sv = vtile_scale(xc);
            advance(xc);
            const int sa = tile_scale(xc);
            if constexpr (decltype(first)::value) softmax_first(nvalid, hook);
            else softmax(nvalid, hook);
            asm volatile("" ::"s"(sa), "s"(sv));
            m_prefetch88(lds + stage_of(t) * SB + KTB);
            wg_barrier();
            m_block88(lds + stage_of(t) * SB + KTB, lds + stage_of(t + 1) * SB, sa, sv, std::true_type{});
          } else if constexpr (KF8) {
            // the next tile's scale is read before the softmax, so its
            // scalar load has returned by the MFMA block
            const int nvalid = xc.n - xc.j0;
            advance(xc);
            const int sa = tile_scale(xc);
            if constexpr (decltype(first)::value) softmax_first(nvalid, hook);
            else softmax(nvalid, hook);
            asm volatile("" ::"s"(sa));
            m_prefetch(lds + stage_of(t) * SB + KTB);
            wg_barrier();
            m_block8(lds + stage_of(t) * SB + KTB, lds + stage_of(t + 1) * SB, sa);
          } else {
            if constexpr (decltype(first)::value) softmax_first(xc.n - xc.j0, hook);
            else softmax(xc.n - xc.j0, hook);
            advance(xc);
            m_prefetch(lds + stage_of(t) * SB + KTB);
            wg_barrier();
            m_block(lds + stage_of(t) * SB + KTB, lds + stage_of(t + 1) * SB,
                    std::true_type{});
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile t+2 (group B's loads) has landed
          wg_barrier();
        };
        using L0 = std::integral_constant<int, 0>;
        using L1 = std::integral_constant<int, 1>;
        if (NP > 1) {
          int t = 1;
          if (group == 1 && NP > 2) {
            period(0, std::true_type{}, L1{});
            for (; t + 2 < NP; ++t) period(t, std::false_type{}, L1{});
          } else {
            period(0, std::true_type{}, L0{});
            for (; t + 2 < NP; ++t) period(t, std::false_type{}, L0{});
          }
          if (t + 1 < NP) period(t, std::false_type{}, L0{});   // t = NP-2: nothing left to load
          softmax(xc.n - xc.j0, no_hook);      // X(NP-1)
        } else {
          softmax_first(xc.n - xc.j0, no_hook);
        }
        if constexpr (VF8) {
          const int sv = vtile_scale(xc);
          m_prefetch88(lds + stage_of(NP - 1) * SB + KTB);
          wg_barrier();
          m_block88(lds + stage_of(NP - 1) * SB + KTB, nullptr, 0, sv, std::false_type{});
        } else {
          m_prefetch(lds + stage_of(NP - 1) * SB + KTB);
          wg_barrier();
          m_block(lds + stage_of(NP - 1) * SB + KTB, nullptr, std::false_type{});
        }
        wg_barrier();
        if (group == 0) wg_barrier();          // match group B's extra leading barrier
      }


    if (!SPLIT || (ka == 0 && kb == NT)) {
      write_out(head, qrow);
      return;
    }
    (void)v;
    (void)j;
    if constexpr (SPLIT) {
      // Part j of cut remainder unit v: its fp32 state (O, m, l in register
      // order) goes to slot j * rU + v; attn_merge_kernel, launched next on
      // the same stream, combines a unit's parts and writes the output.
      constexpr int SLOT = (int)(kSplitSlotBytes / 4), ML = 8 * 64 * 64;
      float* mine = a.part + (size_t)(j * rU + v) * SLOT;
#pragma unroll
      for (int r = 0; r < 64; ++r) mine[(wave * 64 + r) * 64 + lane] = o[r >> 4][r & 15];
      mine[ML + (wave * 2) * 64 + lane] = m_run;
      mine[ML + (wave * 2 + 1) * 64 + lane] = l_run;
    }
  };

  if constexpr (!SPLIT) {
    // one unit per workgroup, XCD-contiguous (the query tiles of a head share an L2)
    const int u = __builtin_amdgcn_readfirstlane(a.unit0 + xcd_remap(blockIdx.x, gridDim.x));
    piece(u, 0, NT, -1, 0);
  } else {
    // kStreamWG workgroups: part p of remainder unit v on workgroup
    // p * rU + v, so the query tiles of a head read the same key part at the
    // same time.
    const int jw = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, kStreamWG));
    if (jw < rU * rP) {
      const int v = jw % rU, p = jw / rU;
      piece(a.unit0 + v, NT * p / rP, NT * (p + 1) / rP, v, p);
    }
  }
}

// Split launch, second step: the rP part states of each cut remainder unit
// (slot p * rU + v holds part p of unit unit0 + v, as the attention kernel's
// lanes held it) are combined in part order, normalised and stored as bf16.
// One wave per (unit, attention wave), i.e. per 32 query rows; the kernel
// boundary after the split launch makes the slots visible.
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a) {
  constexpr int SLOT = (int)(kSplitSlotBytes / 4), ML = 8 * 64 * 64;
  const int nqt = (a.T + ABM - 1) / ABM;
  const int rU = a.H * nqt - a.unit0, rP = a.parts;
  const int v = blockIdx.x >> 3, wave = blockIdx.x & 7, lane = threadIdx.x;
  const int u = a.unit0 + v;
  const int head = u / nqt, qt = u - head * nqt;
  const int qrow = qt * ABM + wave * 32 + (lane & 31), hh = lane >> 5;
  const float* slot0 = a.part + (size_t)v * SLOT;
  const size_t pstride = (size_t)rU * SLOT;
  float mm = -INFINITY;
  for (int p = 0; p < rP; ++p) mm = fmaxf(mm, slot0[p * pstride + ML + (wave * 2) * 64 + lane]);
  float o[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) o[r] = 0.f;
  float l = 0.f;
  for (int p = 0; p < rP; ++p) {
    const float* sp = slot0 + p * pstride;
    // all of the part's loads in flight before the first use
    float t[64];
#pragma unroll
    for (int r = 0; r < 64; ++r) t[r] = sp[(wave * 64 + r) * 64 + lane];
    const float mp = sp[ML + (wave * 2) * 64 + lane];
    const float lp = sp[ML + (wave * 2 + 1) * 64 + lane];
    const float be = mp > -INFINITY ? __builtin_amdgcn_exp2f(mp - mm) : 0.f;
    l += be * lp;
#pragma unroll
    for (int r = 0; r < 64; ++r) o[r] += be * t[r];
  }
  // lanes l and l ^ 32 hold the two halves of a row's sum
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow >= a.T) return;
  __bf16* op = static_cast<__bf16*>(a.out) + ((size_t)qrow * a.H + head) * AD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[16 * db + 4 * j + e] * inv);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hh) = w;
    }
}

// ------------------------------------------------------------------ attention, fp32
// A query's D channels are spread over G = D/8 lanes (8 channels each): a
// score is 8 FMAs per lane and a sum over the G lanes by DPP moves within
// the lanes' row (every lane ends with the same value), and the lanes' 8
// output channels accumulate P V directly.  A workgroup holds the queries
// of one head (key groups below).
//
// Both tiles sit key-major in LDS, so a lane reads its 8 channels of a key
// as two float4: K rows as they are, V transposed from V^T on the way in,
// with the 16-byte chunk q of key row j at q ^ (j & (D/4 - 1)) so that the
// transposing stores (four keys of one channel per lane) spread over the
// banks.  A lane reads chunks c0/4 and c0/4 + 1 of one row, which the XOR
// keeps distinct across the lanes of the row.  The next tile of a segment
// is loaded into registers while the current one is computed.  Logits are
// base 2 (q carries softmax_scale * log2 e).
//
// Sum over aligned groups of G = 8 or 16 lanes: swap neighbours, then pairs,
// then the two quads of each 8 (row_half_mirror), then the two 8s of each
// 16 (row_mirror).  Each step adds a value to its partner's, and fp32
// addition is commutative, so all lanes of a group hold the same sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 8 || G == 16, "groups of 8 or 16 lanes");
  auto dpp = [](float v, auto ctrl_t) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl_t)::value, 0xF, 0xF, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  if constexpr (G == 16) x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
  return x;
}

// Key groups: a workgroup holds KG groups of LG lanes over the same
// queries.  The context's key tiles are numbered in segment order and dealt
// round-robin, tile f to group f mod KG, so each group runs 1/KG of the
// tiles with its own LDS tiles and its own running (m, l, O); at the end
// groups 1..KG-1 hand their states to group 0 through LDS, which combines
// them in group order (m = the largest max, O and l summed with weights
// 2^(m_g - m)) and writes the output.  Every group passes every barrier: a
// round in which a group has no tile left skips only its work.  With D = 64
// a group is one wave of 8 queries and a workgroup 8 groups (two waves per
// SIMD) over key tiles of 32, so that small blocks spread over many CUs;
// D = 128 needs more than half of a SIMD's registers per wave, so it keeps
// one group of 256 lanes (16 queries) and tiles of 64.
template <int D>
__global__ __launch_bounds__(D == 64 ? 512 : 256) void attn_f32_kernel(AttnArgs a) {
  constexpr int G = D / 8;                 // lanes per query
  constexpr int LG = D == 64 ? 64 : 256;   // lanes per key group
  constexpr int QPB = LG / G;              // queries per workgroup
  constexpr int KG = D == 64 ? 8 : 1;      // key groups
  constexpr int BNF = D == 64 ? 32 : 64;   // keys per tile
  constexpr int NC = D / 4;                // 16-byte chunks per key row
  constexpr int NL = BNF * D / 4 / LG;     // float4 loads per lane per operand and tile
  static_assert(KG == 1 || (KG - 1) * 10 * LG <= KG * BNF * D, "the merge states (m, l, 8 O per lane) fit the K tiles");
  __shared__ __attribute__((aligned(16))) float s_k4[KG][BNF][D];
  __shared__ __attribute__((aligned(16))) float s_v4[KG][BNF][D];
  __shared__ const float* s_k[kMaxSeg];
  __shared__ const float* s_v[kMaxSeg];
  __shared__ int s_n[kMaxSeg];
  __shared__ int s_ld[kMaxSeg];
  const int tid = threadIdx.x;
  const int kg = __builtin_amdgcn_readfirstlane(tid / LG);   // key group
  const int gt = tid % LG;                 // lane within the group
  const int nqt = (a.T + QPB - 1) / QPB;
  const int head = blockIdx.x / nqt, qt = blockIdx.x - head * nqt;
  if (tid < a.nseg) {
    const Seg sg = a.seg[tid];
    const char* kb;
    const char* vb;
    long long khs, vhs;
    int ld;
    if (sg.dyn >= 0) {
      const int slot = a.sel_slots[sg.dyn];
      kb = a.slot_base + (long long)slot * a.slot_bytes;
      vb = kb + a.slot_v_off;
      khs = a.slot_k_hs;
      vhs = a.slot_v_hs;
      ld = a.slot_v_ld;
      if (sg.k) {                        // K rotated into the context-K buffer
        kb = static_cast<const char*>(sg.k);
        khs = sg.k_hs;
      }
    } else {
      kb = static_cast<const char*>(sg.k);
      vb = static_cast<const char*>(sg.v);
      khs = sg.k_hs;
      vhs = sg.v_hs;
      ld = sg.v_ld;
    }
    s_k[tid] = reinterpret_cast<const float*>(kb) + head * khs;
    s_v[tid] = reinterpret_cast<const float*>(vb) + head * vhs;
    s_n[tid] = sg.n;
    s_ld[tid] = ld;
  }
  const int sub = gt % G, c0 = 8 * sub;    // this lane's channels c0 .. c0 + 7
  const int qrow = qt * QPB + gt / G;
  const bool valid = qrow < a.T;
  float q[8], o[8];
  {
    int f = 0, y = 0, x = 0;
    if (valid) token_fyx(qrow, a.rope.grid_h, a.rope.grid_w, f, y, x);
    const float* qp = static_cast<const float*>(a.q) + ((size_t)(valid ? qrow : 0) * a.H + head) * D + c0;
#pragma unroll
    for (int c = 0; c < 8; ++c) q[c] = valid ? qp[c] : 0.f;
    if (valid && has_rope(a.rope)) {
#pragma unroll
      for (int c = 0; c < 8; c += 2) rope_pair(q[c], q[c + 1], c0 + c, a.rope, a.t_row0 + f, y, x);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      q[c] *= a.qscale;
      o[c] = 0.f;
    }
  }
  __syncthreads();

  float (*const tk)[D] = s_k4[kg];
  float (*const tv)[D] = s_v4[kg];
  // a tile's K rows and V^T columns as float4 loads into registers; keys
  // past nv are not read and enter as 0
  float4 kl[NL], vl[NL];
  auto load_tile = [&](const float* kb, const float* vb, int ld, int j0, int nv) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int idx = it * LG + gt;
      const int r = idx / NC, c4 = idx - r * NC;
      kl[it] = r < nv ? *reinterpret_cast<const float4*>(kb + (size_t)(j0 + r) * D + 4 * c4)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      const int d = idx / (BNF / 4), jj = 4 * (idx - d * (BNF / 4));
      const float* vp = vb + (size_t)d * ld + j0 + jj;
      if (jj + 3 < nv) {
        vl[it] = *reinterpret_cast<const float4*>(vp);
      } else {
        vl[it].x = jj < nv ? vp[0] : 0.f;
        vl[it].y = jj + 1 < nv ? vp[1] : 0.f;
        vl[it].z = jj + 2 < nv ? vp[2] : 0.f;
        vl[it].w = 0.f;
      }
    }
  };
  // chunk position of 16-byte chunk q of key row j
  auto cpos = [](int j, int qc) { return (qc ^ (j & (NC - 1))) * 4; };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int idx = it * LG + gt;
      const int r = idx / NC, c4 = idx - r * NC;
      *reinterpret_cast<float4*>(&tk[r][cpos(r, c4)]) = kl[it];
      const int d = idx / (BNF / 4), jj = 4 * (idx - d * (BNF / 4));
      const int qd = d >> 2, e = d & 3;
      tv[jj][cpos(jj, qd) + e] = vl[it].x;
      tv[jj + 1][cpos(jj + 1, qd) + e] = vl[it].y;
      tv[jj + 2][cpos(jj + 2, qd) + e] = vl[it].z;
      tv[jj + 3][cpos(jj + 3, qd) + e] = vl[it].w;
    }
  };
  // tile cursor in segment order: (segment, first key); sg == nseg past the end
  const int nseg = a.nseg;
  auto skip_empty = [&](int& sg, int& j0) {
    while (sg < nseg && j0 >= s_n[sg]) {
      ++sg;
      j0 = 0;
    }
  };
  auto advance = [&](int& sg, int& j0, int k) {     // k tiles on
    for (int i = 0; i < k && sg < nseg; ++i) {
      j0 += BNF;
      skip_empty(sg, j0);
    }
  };
  int ntiles = 0;                          // context tiles, all segments
  for (int g = 0; g < nseg; ++g) ntiles += (s_n[g] + BNF - 1) / BNF;
  const int rounds = (ntiles + KG - 1) / KG;

  int csg = 0, cj0 = 0;                    // this group's tile of the current round
  skip_empty(csg, cj0);
  advance(csg, cj0, kg);
  if (csg < nseg) load_tile(s_k[csg], s_v[csg], s_ld[csg], cj0, min(BNF, s_n[csg] - cj0));

  float m_run = -INFINITY, l_run = 0.f;
  for (int r = 0; r < rounds; ++r) {
    const bool have = csg < nseg;
    const int nv = have ? min(BNF, s_n[csg] - cj0) : 0;
    if (have) store_tile();
    __syncthreads();
    int nsg = csg, nj0 = cj0;              // the group's tile of the next round
    advance(nsg, nj0, KG);
    if (nsg < nseg) load_tile(s_k[nsg], s_v[nsg], s_ld[nsg], nj0, min(BNF, s_n[nsg] - nj0));   // in flight meanwhile
    if (have) {
      float s[BNF];
      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < BNF; ++jj) {
        const float4 k0 = *reinterpret_cast<const float4*>(&tk[jj][cpos(jj, c0 / 4)]);
        const float4 k1 = *reinterpret_cast<const float4*>(&tk[jj][cpos(jj, c0 / 4 + 1)]);
        float acc = q[0] * k0.x;
        acc = fmaf(q[1], k0.y, acc);
        acc = fmaf(q[2], k0.z, acc);
        acc = fmaf(q[3], k0.w, acc);
        acc = fmaf(q[4], k1.x, acc);
        acc = fmaf(q[5], k1.y, acc);
        acc = fmaf(q[6], k1.z, acc);
        acc = fmaf(q[7], k1.w, acc);
        acc = group_sum<G>(acc);
        s[jj] = (jj < nv) ? acc : -INFINITY;
        mx = fmaxf(mx, s[jj]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] *= alpha;
#pragma unroll
      for (int jj = 0; jj < BNF; ++jj) {
        const float p = __builtin_amdgcn_exp2f(s[jj] - m_new);
        l_run += p;
        const float4 v0 = *reinterpret_cast<const float4*>(&tv[jj][cpos(jj, c0 / 4)]);
        const float4 v1 = *reinterpret_cast<const float4*>(&tv[jj][cpos(jj, c0 / 4 + 1)]);
        o[0] = fmaf(p, v0.x, o[0]);
        o[1] = fmaf(p, v0.y, o[1]);
        o[2] = fmaf(p, v0.z, o[2]);
        o[3] = fmaf(p, v0.w, o[3]);
        o[4] = fmaf(p, v1.x, o[4]);
        o[5] = fmaf(p, v1.y, o[5]);
        o[6] = fmaf(p, v1.z, o[6]);
        o[7] = fmaf(p, v1.w, o[7]);
      }
    }
    __syncthreads();
    csg = nsg;
    cj0 = nj0;
  }
  if constexpr (KG > 1) {
    // groups 1..KG-1 store (m, l, O) per lane in the tile memory the last
    // barrier freed; group 0 combines all KG states in group order
    float* st = &s_k4[0][0][0];
    constexpr int SW = 10 * LG;            // floats per group state
    if (kg > 0) {
      float* sg = st + (kg - 1) * SW;
      sg[gt] = m_run;
      sg[LG + gt] = l_run;
#pragma unroll
      for (int c = 0; c < 8; ++c) sg[(2 + c) * LG + gt] = o[c];
    }
    __syncthreads();
    if (kg != 0) return;
    float m = m_run;
#pragma unroll
    for (int g = 1; g < KG; ++g) m = fmaxf(m, st[(g - 1) * SW + gt]);
    const float a0 = m_run > -INFINITY ? __builtin_amdgcn_exp2f(m_run - m) : 0.f;
    l_run *= a0;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= a0;
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const float* sg = st + (g - 1) * SW;
      const float mg = sg[gt];
      const float ag = mg > -INFINITY ? __builtin_amdgcn_exp2f(mg - m) : 0.f;
      l_run += sg[LG + gt] * ag;
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] += sg[(2 + c) * LG + gt] * ag;
    }
  }
  if (valid) {
    const float inv = 1.f / l_run;
    float* op = static_cast<float*>(a.out) + ((size_t)qrow * a.H + head) * D + c0;
#pragma unroll
    for (int c = 0; c < 8; ++c) op[c] = o[c] * inv;
  }
}

// ------------------------------------------------------------------ ConvKV gather
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = D / VEC;
  const GatherPart p = a.part[blockIdx.z];
  const int head = blockIdx.y;
  const int tile0 = blockIdx.x * 64;
  if (tile0 >= p.n) return;
  const int ntok = min(64, p.n - tile0);
  const bool rope = has_rope(a.rope);
  const void* src = p.src;
  long long src_hs = p.src_hs;
  int t_row0 = p.t_row0;
  if (p.dyn >= 0) {     // retrieved block: its slot, and its place among the retrieved by stream id
    src = a.slot_base + (long long)a.sel_slots[p.dyn] * a.slot_bytes;
    src_hs = a.slot_k_hs;
    const int id = a.sel_ids[p.dyn];
    int rank = 0;
    for (int j = 0; j < a.n_dyn; ++j) rank += a.sel_ids[j] < id;
    t_row0 += rank * a.frames;
  }
  // every chunk's load first, then the rotations, then the stores: IT
  // independent 16-byte loads in flight per thread (rows past the tail load
  // the tile's last row and are not stored, so no load sits in a branch)
  constexpr int IT = 64 * CPR / 256;
  static_assert(IT * 256 == 64 * CPR, "tile of 64 rows in whole passes of 256 threads");
  const T* sbase = static_cast<const T*>(src) + head * src_hs;
  // the table loads first (cache hits), then the rows, all in flight together
  float2 cs[IT][VEC / 2];
  if (rope) {
    const RopeSel rs(a.rope);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = threadIdx.x + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
      int f, y, x;
      token_fyx(tile0 + r, a.rope.grid_h, a.rope.grid_w, f, y, x);
#pragma unroll
      for (int e = 0; e < VEC; e += 2) cs[it][e / 2] = rs.cs(c * VEC + e, t_row0 + f, y, x);
    }
  }
  uint4 raw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = threadIdx.x + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
    raw[it] = *reinterpret_cast<const uint4*>(sbase + (size_t)(tile0 + r) * D + c * VEC);
  }
  if (rope) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      T* kv = reinterpret_cast<T*>(&raw[it]);
#pragma unroll
      for (int e = 0; e < VEC; e += 2) {
        float u0 = to_f(kv[e]), u1 = to_f(kv[e + 1]);
        rope_rot(u0, u1, cs[it][e / 2]);
        kv[e] = from_f<T>(u0);
        kv[e + 1] = from_f<T>(u1);
      }
    }
  }
  T* dbase = static_cast<T*>(a.dst) + head * a.dst_hs + (size_t)(p.dst_off + tile0) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = threadIdx.x + 256 * it, r = task / CPR, c = task % CPR;
    if (r < ntok) *reinterpret_cast<uint4*>(dbase + (size_t)r * D + c * VEC) = raw[it];
  }
}

// FP8 keys: the same gather into E4M3 rows.  One workgroup = one 64-row tile
// of one head of one part: rotate in fp32, reduce the tile's largest |K~|,
// store E4M3 with that tile's power-of-two scale and the exponent beside it
// (the append_k8_kernel rule, tiles counted from the segment's first row).
__global__ __launch_bounds__(256) void gather_k8_kernel(GatherArgs a) {
  constexpr int D = 128, VEC = 8, CPR = D / VEC, IT = 64 * CPR / 256;
  __shared__ float s_max[4];
  const GatherPart p = a.part[blockIdx.z];
  const int head = blockIdx.y;
  const int tile0 = blockIdx.x * 64;
  if (tile0 >= p.n) return;
  const int ntok = min(64, p.n - tile0);
  const int tid = threadIdx.x;
  const bool rope = has_rope(a.rope);
  const void* src = p.src;
  long long src_hs = p.src_hs;
  int t_row0 = p.t_row0;
  if (p.dyn >= 0) {
    src = a.slot_base + (long long)a.sel_slots[p.dyn] * a.slot_bytes;
    src_hs = a.slot_k_hs;
    const int id = a.sel_ids[p.dyn];
    int rank = 0;
    for (int j = 0; j < a.n_dyn; ++j) rank += a.sel_ids[j] < id;
    t_row0 += rank * a.frames;
  }
  const __bf16* sbase = static_cast<const __bf16*>(src) + head * src_hs;
  // the table loads first (cache hits), then the rows, all in flight together
  float2 cs[IT][VEC / 2];
  if (rope) {
    const RopeSel rs(a.rope);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
      int f, y, x;
      token_fyx(tile0 + r, a.rope.grid_h, a.rope.grid_w, f, y, x);
#pragma unroll
      for (int e = 0; e < VEC; e += 2) cs[it][e / 2] = rs.cs(c * VEC + e, t_row0 + f, y, x);
    }
  }
  float kr[IT][VEC];
  bf16x8 raw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {   // rows past the tail load the last row (not used)
    const int task = tid + 256 * it, r = min(task / CPR, ntok - 1), c = task % CPR;
    raw[it] = *reinterpret_cast<const bf16x8*>(sbase + (size_t)(tile0 + r) * D + c * VEC);
  }
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR;
    const bool live = r < ntok;           // rows past the tail count as 0
#pragma unroll
    for (int e = 0; e < VEC; ++e) kr[it][e] = live ? (float)raw[it][e] : 0.f;
    if (rope) {
#pragma unroll
      for (int e = 0; e < VEC; e += 2) rope_rot(kr[it][e], kr[it][e + 1], cs[it][e / 2]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) amax = fmaxf(amax, fabsf(kr[it][e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const int ex = e4m3_exponent(amax);
  const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
  char* dbase = static_cast<char*>(a.dst) + head * a.dst_hs + (size_t)(p.dst_off + tile0) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int task = tid + 256 * it, r = task / CPR, c = task % CPR;
    if (r >= ntok) continue;
    uint2 w;
    w.x = (unsigned)e4m3_pack4(kr[it][0] * inv, kr[it][1] * inv, kr[it][2] * inv, kr[it][3] * inv);
    w.y = (unsigned)e4m3_pack4(kr[it][4] * inv, kr[it][5] * inv, kr[it][6] * inv, kr[it][7] * inv);
    *reinterpret_cast<uint2*>(dbase + (size_t)r * D + c * VEC) = w;
  }
  if (tid == 0) a.dx[head * a.dx_hs + p.x_off + blockIdx.x] = ex;
}

// ------------------------------------------------------------------ ConvKV conv
// blockIdx.z = memory frame j, blockIdx.y = 0 (K rows) / 1 (V^T rows).
// mem[j][h][s][c] = sum_i w[h][c][i] * frame[j*kernel + i][h][s][c], fp32 sums
// in tap order.  KS = kernel (taps per memory frame): a thread issues the
// loads of all its taps before the first multiply.
template <typename T, bool VEC_V, int KS>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  const int j = blockIdx.z;
  const int D = a.D, Tf = a.Tf;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.y == 0) {
    // K rows: chunks of VEC channels; index = (h * Tf + s) * (D / VEC) + c
    const int cpr = D / VEC;
    const long long total = (long long)a.H * Tf * cpr;
    if (gid >= total) return;
    const int c = (int)(gid % cpr);
    const long long hs = gid / cpr;
    const int s = (int)(hs % Tf), h = (int)(hs / Tf);
    uint4 raw[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k_src[j * KS + i]) + h * a.k_hs +
                                               (size_t)s * D + c * VEC);
    // the thread's weights w[h][c*VEC + e][i] are VEC * KS consecutive floats
    // (16-byte aligned: VEC * KS * 4 is a multiple of 16)
    constexpr int NW = VEC * KS / 4;
    float4 wq[NW];
    const float4* wsrc = reinterpret_cast<const float4*>(a.wk + ((size_t)h * D + c * VEC) * KS);
#pragma unroll
    for (int q = 0; q < NW; ++q) wq[q] = wsrc[q];
    const float* w = reinterpret_cast<const float*>(wq);
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const T* v = reinterpret_cast<const T*>(&raw[i]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w[e * KS + i], to_f(v[e]), acc[e]);
    }
    uint4 out;
    T* ov = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int e = 0; e < VEC; ++e) ov[e] = from_f<T>(acc[e]);
    T* dst = static_cast<T*>(a.k_mem) + h * a.k_mem_hs + (size_t)(j * a.tf_pad + s) * D + c * VEC;
    *reinterpret_cast<uint4*>(dst) = out;
  } else {
    // V^T rows: index = (h * D + d) * groups + g, groups of VEC tokens
    const int groups = (Tf + VEC - 1) / VEC;
    const long long total = (long long)a.H * D * groups;
    if (gid >= total) return;
    const int g = (int)(gid % groups);
    const long long hd = gid / groups;
    const int d = (int)(hd % D), h = (int)(hd / D);
    const int s0 = g * VEC;
    const int nv = min(VEC, Tf - s0);
    float w[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) w[i] = a.wv[((size_t)h * D + d) * KS + i];
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    if (VEC_V && nv == VEC) {
      uint4 raw[KS];
#pragma unroll
      for (int i = 0; i < KS; ++i)
        raw[i] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.vt_src[j * KS + i]) + h * a.vt_hs +
                                                 (size_t)d * a.vt_ld + s0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const T* v = reinterpret_cast<const T*>(&raw[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(w[i], to_f(v[e]), acc[e]);
      }
    } else {
      for (int i = 0; i < KS; ++i) {
        const T* src = static_cast<const T*>(a.vt_src[j * KS + i]) + h * a.vt_hs + (size_t)d * a.vt_ld + s0;
        for (int e = 0; e < nv; ++e) acc[e] = fmaf(w[i], to_f(src[e]), acc[e]);
      }
    }
    T* dst = static_cast<T*>(a.vt_mem) + h * a.vt_mem_hs + (size_t)d * a.vt_mem_ld + j * a.tf_pad + s0;
    if (nv == VEC) {
      uint4 out;
      T* ov = reinterpret_cast<T*>(&out);
#pragma unroll
      for (int e = 0; e < VEC; ++e) ov[e] = from_f<T>(acc[e]);
      *reinterpret_cast<uint4*>(dst) = out;
    } else {
      for (int e = 0; e < nv; ++e) dst[e] = from_f<T>(acc[e]);
    }
  }
}

// ------------------------------------------------------------------ QKV projection
// out^T = W x^T on v_mfma_f32_32x32x16_bf16: A = 32 rows of W (features) x 16
// channels, B = x^T, 16 channels x 32 tokens, so a lane's accumulator holds
// groups of 4 consecutive features of one token (MFMA rows 8g + 4h .. +3 for
// lane half h) and RoPE's channel pairs never cross lanes.
//
// Workgroup: 256 features x 256 tokens, 8 waves as 2 x 4 (128 features x 64
// tokens each: 4 x 2 blocks of 32 x 32), 32 channels per step.  Both operand
// tiles are rows of 32 channels (64 B) in LDS, chunk c of row r at
// c ^ ((r >> 2) & 3): the 16 rows a 16-lane phase reads (same chunk index)
// then cover the 64 banks once.  Tiles move with buffer_load ... lds, four
// stages deep, three steps ahead.  Only waves 0-3 issue loads (eight per step
// each, four between the MFMAs of each half-step): every load blocks its
// wave until the CU's address unit takes it, so the loads are kept off half
// of the waves and spread over the step.  Rows past the last token or
// feature are loaded clamped to the last valid row and never stored.
constexpr int GF = 256, GT = 256, GK = 32, GSTAGE = 4;
constexpr int G_OPB = GF * GK * 2;          // bytes of one operand tile per step (16 KB)
static_assert(GF == GT, "both operand tiles share the load mapping");

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void qkv_gemm_kernel(QkvArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[GSTAGE * 2 * G_OPB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave >> 2, wt = wave & 3;
  const int hh = lane >> 5, col = lane & 31;
  const int H = a.ap.H, T = a.ap.T, C = a.C;
  const int HD = H * AD, NF = 3 * HD;
  const int ntb = (T + GT - 1) / GT;
  const int u = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, gridDim.x));
  const int fb = u / ntb, tb = u - fb * ntb;
  const int f0 = fb * GF, t0 = tb * GT;

  // loads: chunk p = (8i + wave)*64 + lane of an operand tile (i = 0, 1) lands
  // at LDS p*16 = row 128i + 16 wave + (lane >> 2), position lane & 3, which
  // holds the row's chunk (lane & 3) ^ ((lane >> 4) & 3)
  // waves 0-3 load (each for wave slots w and w + 4); waves 4-7 issue no loads
  const unsigned cpos = (unsigned)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  unsigned vw[2][2], vx[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int rl = 16 * ((wave & 3) + 4 * k) + (lane >> 2);
      vw[i][k] = (unsigned)min(f0 + 128 * i + rl, NF - 1) * (unsigned)C * 2u + cpos;
      vx[i][k] = (unsigned)min(t0 + 128 * i + rl, T - 1) * (unsigned)C * 2u + cpos;
    }
  const bool loader = wave < 4;
  const i32x4 rw = buffer_rsrc(uniform_ptr(a.w)), rx = buffer_rsrc(uniform_ptr(a.x));
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_ptr_t)lds;
  const int S = C / GK;
  // load j (0..7) of step s: operand j >> 2 (W, x), i = (j >> 1) & 1, slot k = j & 1
  auto issue_one = [&](int s, int j) {       // loading waves only
    const unsigned base = __builtin_amdgcn_readfirstlane(lds0 + (unsigned)(s & (GSTAGE - 1)) * 2 * G_OPB);
    const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)s * GK * 2u);
    const int i = (j >> 1) & 1, k = j & 1, w = (wave & 3) + 4 * k;
    if (j < 4) dma16(rw, vw[i][k], soff, base + (8 * i + w) * 1024);
    else dma16(rx, vx[i][k], soff, base + G_OPB + (8 * i + w) * 1024);
  };
  auto issue = [&](int s) {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_one(s, j);
  };
  auto frag = [&](const char* tile, int row, int c) {
    return *reinterpret_cast<const bf16x8*>(tile + row * 64 + ((c ^ ((row >> 2) & 3)) << 4));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) acc[bm][bn] = f32x16{};

  // Fragments of half-step (s, ss) are read one half-step ahead of their
  // MFMAs.  Step s+1 is published by a barrier between the two halves of step
  // s, which each wave reaches with its chunks of step s+1 landed and all its
  // LDS reads returned; the first reads of s+1 then overlap the MFMAs of
  // (s, 1).  The reads of step s-1 end before the barrier of step s-1, so
  // from there on step s+3 may refill that buffer: its loads go in during
  // both halves of step s.
  auto read_half = [&](int s, int ss, bf16x8 (&af)[4], bf16x8 (&bx)[2]) {
    const char* A = lds + (s & (GSTAGE - 1)) * 2 * G_OPB;
    const char* B = A + G_OPB;
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) af[bm] = frag(A, 128 * wf + 32 * bm + col, 2 * ss + hh);
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) bx[bn] = frag(B, 64 * wt + 32 * bn + col, 2 * ss + hh);
  };
  // eight MFMAs; with loads (a compile-time choice: loading waves, steps
  // with a step left to load), loads load_j0 .. load_j0 + 3 of load_step go
  // in after MFMAs 1, 3, 5, 7
  auto mfma_half = [&](const bf16x8 (&af)[4], const bf16x8 (&bx)[2], int load_step, int load_j0, auto loads) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], bx[bn], acc[bm][bn], 0, 0, 0);
        if constexpr (decltype(loads)::value) {
          if (bn == 1) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(load_step, load_j0 + bm);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
  };
  bf16x8 a0[4], b0[2], a1[4], b1[2];
  if (loader) {
    issue(0);
    if (S > 1) issue(1);
    if (S > 2) issue(2);
  }
  // this wave's chunks of step 0 have landed
  if (S > 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (S > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  wg_barrier();
  read_half(0, 0, a0, b0);
  // step s; with_loads: step s+3 exists and this wave loads (the steady
  // steps of a loading wave: no run-time test around any load)
  auto step = [&](int s, auto with_loads) {
    read_half(s, 1, a1, b1);
    mfma_half(a0, b0, s + 3, 0, with_loads);
    if (s + 1 < S) {
      // this wave's chunks of step s+1 have landed (step s+2 may be in flight)
      // loads after step s+1's: step s+2 (8) and the first 4 of step s+3
      if (s + 3 < S) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
      else if (s + 2 < S) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      wg_barrier();
      read_half(s + 1, 0, a0, b0);
    }
    mfma_half(a1, b1, s + 3, 4, with_loads);
  };
  int s = 0;
  if (loader)
    for (; s + 3 < S; ++s) step(s, std::true_type{});
  for (; s < S; ++s) step(s, std::false_type{});

  // epilogue: + bias; q -> scratch [T][H][D]; k -> (raw copy,) RoPE -> cache
  // rows; v -> V^T.  A wave's 128 features are one head of one of q, k, v
  // (f0 is a multiple of 256 and a head is 128 features), so which and head
  // are wave-uniform.
  // Loads come before stores: the compiler cannot move a load above a store
  // that may alias it, so a bias or RoPE table load placed between stores
  // waits out its whole latency, once per load.  For each token column and
  // 32-feature block (bn, bm), the bias (4 values per group g) and the RoPE
  // (cos, sin) of the block's 8 channel pairs are loaded together, then the
  // block's 4 groups are formed and stored.
  const AppendArgs& ap = a.ap;
  const bool rope = has_rope(ap.rope);
  const __bf16* bias = static_cast<const __bf16*>(a.b);
  const int fw = f0 + 128 * wf, tw = t0 + 64 * wt;
  if (fw >= NF || tw >= T) return;         // rows past the last feature or token: never stored
  const int which = fw / HD, head = (fw - which * HD) / AD;
  const RopeSel rs(ap.rope);
  const bool rot = which == 1 && rope;
  int fyx[2][3];                           // (frame, y, x) of the token columns, clamped into the block
#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
    token_fyx(min(tw + 32 * bn + col, T - 1), ap.rope.grid_h, ap.rope.grid_w, fyx[bn][0], fyx[bn][1], fyx[bn][2]);
  bf16x4 bb[4];                            // bias of the block's groups
  float2 cs[4][2];                         // (cos, sin) of channel pairs d0, d0 + 2 of each group
  auto load_block = [&](int bn, int bm) {
    if (bias) {
#pragma unroll
      for (int g = 0; g < 4; ++g) bb[g] = *reinterpret_cast<const bf16x4*>(bias + fw + 32 * bm + 8 * g + 4 * hh);
    }
    if (rot) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2)
          cs[g][p2] = rs.cs(32 * bm + 8 * g + 4 * hh + 2 * p2, ap.t_row0 + fyx[bn][0], fyx[bn][1], fyx[bn][2]);
    }
  };
  // value j of group (bm, g) for token column bn: + bias, rounded to bf16 as
  // it leaves the projection (as the unfused path receives it)
  auto value4 = [&](int bm, int bn, int g, float (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[bm][bn][4 * g + j];
    if (bias) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += (float)bb[g][j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (float)(__bf16)v[j];
  };
  // FP8 caches: a wave's 128 features x 64 tokens are one head's K (or V)
  // over one 64-token tile of the block (both aligned), so the tile's scale
  // is a reduction within the wave.  Pass 1 forms every value (bias, bf16
  // rounding, the raw copies, RoPE for K) and reduces the largest magnitude
  // over the valid tokens; pass 2 forms the values again and stores E4M3
  // bytes and the tile exponent.  Forming them twice keeps the accumulators
  // as they are, which keeps the epilogue free of register spills.
  if ((ap.k8 && which == 1) || (ap.v8 && which == 2)) {
    const bool isk = which == 1;
    float amax = 0.f;
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
      const int t = tw + 32 * bn + col;
      const bool live = t < T;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        load_block(bn, bm);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * bm + 8 * g + 4 * hh;
          float v[4];
          value4(bm, bn, g, v);
          if (live) {
            if (isk && ap.k_raw) {
              bf16x4 o;
#pragma unroll
              for (int j = 0; j < 4; ++j) o[j] = (__bf16)v[j];
              *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(ap.k_raw) + head * ap.k_raw_hs + (size_t)t * AD + d0) = o;
            } else if (!isk && ap.vt) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                static_cast<__bf16*>(ap.vt)[head * ap.vt_hs + (size_t)(d0 + j) * ap.vt_ld + t] = (__bf16)v[j];
            }
          }
          if (rot) {
            rope_rot(v[0], v[1], cs[g][0]);
            rope_rot(v[2], v[3], cs[g][1]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) amax = live ? fmaxf(amax, fabsf(v[j])) : amax;
          asm volatile("" : "+v"(amax));   // reduce here: the group's values die now
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const int ex = e4m3_exponent(amax);
    const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
    // pass 2: the values again, stored as E4M3 with the tile's scale
#pragma unroll
    for (int bn = 0; bn < 2; ++bn) {
      const int t = tw + 32 * bn + col;
      const bool live = t < T;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        load_block(bn, bm);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * bm + 8 * g + 4 * hh;
          float v[4];
          value4(bm, bn, g, v);
          if (rot) {
            rope_rot(v[0], v[1], cs[g][0]);
            rope_rot(v[2], v[3], cs[g][1]);
          }
          const int w = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
          if (live) {
            if (isk) {
              *reinterpret_cast<int*>(static_cast<char*>(ap.k8) + head * ap.k8_hs + (size_t)t * AD + d0) = w;
            } else {
              unsigned char* vp = static_cast<unsigned char*>(ap.v8) + head * ap.v8_hs + t;
#pragma unroll
              for (int j = 0; j < 4; ++j) vp[(size_t)(d0 + j) * ap.v8_ld] = (unsigned char)(w >> (8 * j));
            }
          }
        }
      }
    }
    if (lane == 0) {
      if (isk) ap.kx[head * ap.kx_hs + tw / 64] = ex;
      else ap.vx[head * ap.vx_hs + tw / 64] = ex;
    }
    return;                                // this wave held K (or V) of the FP8 cache only
  }
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    const int t = tw + 32 * bn + col;
    const bool live = t < T;
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      load_block(bn, bm);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * bm + 8 * g + 4 * hh;
        float v[4];
        value4(bm, bn, g, v);
        if (!live) continue;
        bf16x4 o;
        if (which == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = (__bf16)v[j];
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.q) + ((size_t)t * H + head) * AD + d0) = o;
        } else if (which == 1) {
          // the rotation starts from the bf16 value k leaves the projection with
          if (ap.k_raw) {
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = (__bf16)v[j];
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(ap.k_raw) + head * ap.k_raw_hs + (size_t)t * AD + d0) = o;
          }
          if (rot) {
            rope_rot(v[0], v[1], cs[g][0]);
            rope_rot(v[2], v[3], cs[g][1]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = (__bf16)v[j];
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(ap.k_rot) + head * ap.k_rot_hs +
                                     (size_t)(ap.k_rot_off + t) * AD + d0) = o;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            static_cast<__bf16*>(ap.vt)[head * ap.vt_hs + (size_t)(d0 + j) * ap.vt_ld + t] = (__bf16)v[j];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ FP8 V^T of a bf16 V^T
// One workgroup per (64-token tile, head): the tile's 128 rows of 64 bf16
// values (16 KiB) are loaded 16 bytes per chunk, the largest magnitude is
// reduced over the workgroup, and each chunk is written back as 8 E4M3 bytes
// with the tile's power-of-two scale (the append kernel's rule); the tile
// exponent goes beside the rows.  Pad columns hold 0 in the source and stay
// 0.
__global__ __launch_bounds__(256) void vquant_kernel(VQuantArgs a) {
  __shared__ float s_max[4];
  const int tile0 = blockIdx.x * 64, head = blockIdx.y, tid = threadIdx.x;
  const char* src = static_cast<const char*>(a.vt) + 2 * (head * a.vt_hs + tile0);
  bf16x8 raw[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {          // chunk c = tid + 256 it: row c >> 3, 8 tokens (c & 7) * 8
    const int c = tid + 256 * it;
    raw[it] = *reinterpret_cast<const bf16x8*>(src + (size_t)(c >> 3) * a.vt_ld * 2 + (c & 7) * 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[it][e]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const int ex = e4m3_exponent(amax);
  const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
  char* dst = static_cast<char*>(a.v8) + head * a.v8_hs + tile0;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;
    uint2 w;
    w.x = (unsigned)e4m3_pack4((float)raw[it][0] * inv, (float)raw[it][1] * inv, (float)raw[it][2] * inv,
                               (float)raw[it][3] * inv);
    w.y = (unsigned)e4m3_pack4((float)raw[it][4] * inv, (float)raw[it][5] * inv, (float)raw[it][6] * inv,
                               (float)raw[it][7] * inv);
    *reinterpret_cast<uint2*>(dst + (size_t)(c >> 3) * a.v8_ld + (c & 7) * 8) = w;
  }
  if (tid == 0) a.vx[head * a.vx_hs + blockIdx.x] = ex;
}

// ------------------------------------------------------------------ export
template <typename T>
__global__ void export_kernel(ExportArgs a) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)a.seg.n * a.H * a.D;
  if (gid >= total) return;
  const int d = (int)(gid % a.D);
  const long long th = gid / a.D;
  const int h = (int)(th % a.H);
  const int tok = (int)(th / a.H);
  const char* kb;
  const char* vb;
  long long khs, vhs;
  int ld;
  if (a.seg.dyn >= 0) {
    const int slot = a.sel_slots[a.seg.dyn];
    kb = a.slot_base + (long long)slot * a.slot_bytes;
    vb = kb + a.slot_v_off;
    khs = a.slot_k_hs;
    vhs = a.slot_v_hs;
    ld = a.slot_v_ld;
    if (a.seg.k) {                       // K rotated into the context-K buffer
      kb = static_cast<const char*>(a.seg.k);
      khs = a.seg.k_hs;
    }
  } else {
    kb = static_cast<const char*>(a.seg.k);
    vb = static_cast<const char*>(a.seg.v);
    khs = a.seg.k_hs;
    vhs = a.seg.v_hs;
    ld = a.seg.v_ld;
  }
  if constexpr (std::is_same<T, __bf16>::value) {
    if (a.vf8) {   // E4M3 byte times 2^(tile exponent): exact in bf16
      const bool in_slot = a.seg.dyn >= 0;
      const int* xb = in_slot ? reinterpret_cast<const int*>(a.slot_base + (long long)a.sel_slots[a.seg.dyn] *
                                                              a.slot_bytes + a.slot_vx_off)
                              : a.seg.vx;
      const long long xhs = in_slot ? a.slot_vx_hs : a.seg.vx_hs;
      const int byte = reinterpret_cast<const unsigned char*>(vb)[h * vhs + (size_t)d * ld + tok];
      static_cast<T*>(a.v_out)[gid] =
          (T)__builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(byte, 0), xb[h * xhs + tok / 64]);
    } else {
      static_cast<T*>(a.v_out)[gid] = reinterpret_cast<const T*>(vb)[h * vhs + (size_t)d * ld + tok];
    }
  } else {
    static_cast<T*>(a.v_out)[gid] = reinterpret_cast<const T*>(vb)[h * vhs + (size_t)d * ld + tok];
  }
  if constexpr (std::is_same<T, __bf16>::value) {
    if (a.kf8) {   // E4M3 byte times 2^(tile exponent): exact in bf16
      const bool in_slot = a.seg.dyn >= 0 && !a.seg.k;
      const int* xb = in_slot ? reinterpret_cast<const int*>(kb + a.slot_kx_off) : a.seg.kx;
      const long long xhs = in_slot ? a.slot_kx_hs : a.seg.kx_hs;
      const int byte = reinterpret_cast<const unsigned char*>(kb)[h * khs + (size_t)tok * a.D + d];
      const float kv = __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(byte, 0), xb[h * xhs + tok / 64]);
      static_cast<T*>(a.k_out)[gid] = (T)kv;
      return;
    }
  }
  const T* k = reinterpret_cast<const T*>(kb) + h * khs + (size_t)tok * a.D + d;
  static_cast<T*>(a.k_out)[gid] = *k;
}

}  // namespace

// ------------------------------------------------------------------ launchers
hipError_t launch_rope_table(float2* tab, int rows, int dim, long long pos0, double theta,
                             hipStream_t s) {
  const int half = dim / 2;
  const int n = rows * half;
  if (n <= 0) return hipSuccess;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(tab, rows, half, dim, pos0, theta);
  return hipGetLastError();
}

hipError_t launch_open(const OpenArgs& a, hipStream_t s) {
  open_kernel<<<1, kOpenThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, bool bf16, hipStream_t s) {
  dim3 grid((a.T + 63) / 64, a.H);
  if (a.k8) {
    if (!bf16 || a.D != 128 || !(a.vt || (a.v8 && a.vx))) return hipErrorInvalidValue;
    append_k8_kernel<<<grid, 256, 0, s>>>(a);
  } else if (bf16) {
    if (a.D != 128) return hipErrorInvalidValue;
    append_kernel<__bf16, 128><<<grid, 256, 0, s>>>(a);
  } else if (a.D == 64) {
    append_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  } else if (a.D == 128) {
    append_kernel<float, 128><<<grid, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qkv(const QkvArgs& a, hipStream_t s) {
  if (a.ap.D != AD || a.C <= 0 || a.C % GK != 0 || !(a.ap.k_rot || (a.ap.k8 && a.ap.kx)) ||
      !(a.ap.vt || (a.ap.v8 && a.ap.vx && a.ap.k8)) || !a.q)
    return hipErrorInvalidValue;
  // the tiles are addressed by 32-bit buffer offsets
  if (3LL * a.ap.H * AD * a.C * 2 >= (1LL << 32) || (long long)a.ap.T * a.C * 2 >= (1LL << 32))
    return hipErrorInvalidValue;
  const int nf = (3 * a.ap.H * AD + GF - 1) / GF, nt = (a.ap.T + GT - 1) / GT;
  qkv_gemm_kernel<<<nf * nt, 512, 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ static split slots
// The split launch's part states (O, m, l of each key part) for the
// allocation-free attend: a file-scope device array.  Host code uses only
// the address hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in there), kept per device.
static __device__ __align__(256) float scratch[kStaticSplitBytes / sizeof(float)];

hipError_t static_split_slots(float** slots) {
  constexpr int kMaxDevices = 64;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *slots = addr[dev];
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t s) {
  if (bf16) {
    if (a.D != AD) return hipErrorInvalidValue;
    // One unit per workgroup unless whole-unit rounds would leave more than
    // 15% of kStreamWG workgroup slots idle (and the workspace has split
    // slots).  Then the whole rounds run as a plain launch, the remainder
    // units, cut into key parts, as a second launch, and a third merges the
    // parts.
    const int units = ((a.T + ABM - 1) / ABM) * a.H;
    const bool split = attention_split(a.T, a.H, a.split != 0);
    AttnArgs b = a;
    b.unit0 = 0;
    const int plain = split ? units / kStreamWG * kStreamWG : units;
    if (a.vf8 && !a.kf8) return hipErrorInvalidValue;
    if (plain > 0) {
      if (a.vf8) attn_bf16_kernel<false, true, true><<<plain, 64 * AWAVES, 0, s>>>(b);
      else if (a.kf8) attn_bf16_kernel<false, true, false><<<plain, 64 * AWAVES, 0, s>>>(b);
      else attn_bf16_kernel<false, false, false><<<plain, 64 * AWAVES, 0, s>>>(b);
    }
    if (split) {
      // remainder units rU, each cut into rP key parts of at least one tile
      int NT = 0;
      for (int g = 0; g < a.nseg; ++g) NT += (a.seg[g].n + 63) / 64;
      const int rU = units - plain;
      if (NT < 1 || rU < 1 || rU >= kStreamWG) return hipErrorInvalidValue;
      b.unit0 = plain;
      b.parts = NT < kStreamWG / rU ? NT : kStreamWG / rU;
      if (a.vf8) attn_bf16_kernel<true, true, true><<<kStreamWG, 64 * AWAVES, 0, s>>>(b);
      else if (a.kf8) attn_bf16_kernel<true, true, false><<<kStreamWG, 64 * AWAVES, 0, s>>>(b);
      else attn_bf16_kernel<true, false, false><<<kStreamWG, 64 * AWAVES, 0, s>>>(b);
      if (b.parts > 1) attn_merge_kernel<<<rU * AWAVES, 64, 0, s>>>(b);
    }
  } else if (a.D == 64) {
    const int nwg = ((a.T + 7) / 8) * a.H;             // 8 queries per workgroup
    attn_f32_kernel<64><<<nwg, 512, 0, s>>>(a);        // 8 key groups of one wave
  } else if (a.D == 128) {
    const int nwg = ((a.T + 15) / 16) * a.H;
    attn_f32_kernel<128><<<nwg, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, bool bf16, hipStream_t s) {
  if (a.nparts == 0) return hipSuccess;
  dim3 grid((a.max_n + 63) / 64, a.H, a.nparts);
  if (a.kf8) {
    if (!bf16 || a.D != 128 || !a.dx) return hipErrorInvalidValue;
    gather_k8_kernel<<<grid, 256, 0, s>>>(a);
  } else if (bf16) {
    if (a.D != 128) return hipErrorInvalidValue;
    gather_kernel<__bf16, 128><<<grid, 256, 0, s>>>(a);
  } else if (a.D == 64) {
    gather_kernel<float, 64><<<grid, 256, 0, s>>>(a);
  } else if (a.D == 128) {
    gather_kernel<float, 128><<<grid, 256, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KS>
static void conv_launch(const ConvArgs& a, bool bf16, bool vec_v, dim3 grid, hipStream_t s) {
  if (bf16) {
    if (vec_v) conv_kernel<__bf16, true, KS><<<grid, 256, 0, s>>>(a);
    else conv_kernel<__bf16, false, KS><<<grid, 256, 0, s>>>(a);
  } else {
    if (vec_v) conv_kernel<float, true, KS><<<grid, 256, 0, s>>>(a);
    else conv_kernel<float, false, KS><<<grid, 256, 0, s>>>(a);
  }
}

hipError_t launch_conv(const ConvArgs& a, bool bf16, hipStream_t s) {
  const int vec = bf16 ? 8 : 4;
  const long long nk = (long long)a.H * a.Tf * (a.D / vec);
  const long long nv = (long long)a.H * a.D * ((a.Tf + vec - 1) / vec);
  const long long n = nk > nv ? nk : nv;
  dim3 grid((unsigned)((n + 255) / 256), 2, a.n_mem);
  const size_t esz = bf16 ? 2 : 4;
  const bool vec_v = ((size_t)a.Tf * esz) % 16 == 0;
  switch (a.kernel) {
    case 1: conv_launch<1>(a, bf16, vec_v, grid, s); break;
    case 2: conv_launch<2>(a, bf16, vec_v, grid, s); break;
    case 3: conv_launch<3>(a, bf16, vec_v, grid, s); break;
    case 4: conv_launch<4>(a, bf16, vec_v, grid, s); break;
    case 5: conv_launch<5>(a, bf16, vec_v, grid, s); break;
    case 6: conv_launch<6>(a, bf16, vec_v, grid, s); break;
    case 7: conv_launch<7>(a, bf16, vec_v, grid, s); break;
    case 8: conv_launch<8>(a, bf16, vec_v, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Sustained-rate probe: 8 independent accumulator chains per wave, operands
// in registers, no memory traffic in the loop.  The operands are
// full-mantissa pseudo-random values in [-2, 2) (a multiplicative hash of the
// thread and element), since the matrix core's power -- and so the clock it
// sustains -- depends on the data.  The sum is written only if it is NaN,
// which finite operands cannot produce, so the work stays live.
__global__ __launch_bounds__(512) void mfma_probe_kernel(float* sink, int iters) {
  bf16x8 x, y;
  const unsigned t = blockIdx.x * 512u + threadIdx.x;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned hx = (t * 2654435761u) ^ ((unsigned)e * 2246822519u);
    const unsigned hy = (t * 3266489917u) ^ ((unsigned)e * 668265263u);
    x[e] = (__bf16)((float)(int)((hx >> 8) & 0xffff) / 16384.f - 2.f);
    y[e] = (__bf16)((float)(int)((hy >> 8) & 0xffff) / 16384.f - 2.f);
  }
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (s != s) sink[0] = s;
}

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t s) {
  mfma_probe_kernel<<<workgroups, 512, 0, s>>>(sink, iters);
  return hipGetLastError();
}

hipError_t launch_vquant(const VQuantArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  vquant_kernel<<<dim3((a.n + 63) / 64, a.H), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_export(const ExportArgs& a, bool bf16, hipStream_t s) {
  const long long n = (long long)a.seg.n * a.H * a.D;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (bf16) export_kernel<__bf16><<<blocks, 256, 0, s>>>(a);
  else export_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bkv
