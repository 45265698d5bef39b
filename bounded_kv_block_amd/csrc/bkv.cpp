// C-ABI of the bounded-KV block attention library: config validation,
// workspace layout, call-order state machine and kernel launches.
// The operations follow the PR-Sink description (LiveAnimate page, section 方法)
// and the ConvKV Memory description (SoulX-LiveAct page, section 技术内核); the
// exported calls and their contracts are documented in include/bkv.h.
#include "bkv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "schedule.hpp"

namespace {

thread_local std::string g_err;

bkv_status fail(bkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bkv_status fail(bkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Pose-aware bank replacement (decided on the device): spare slots that let
// blocks open while displaced members are still being read back, and the
// ring of readbacks in flight.
constexpr int kPoseSpare = 2;
constexpr int kPoseRing = 4;

struct Layout {
  int T, Tpad, Tf, tf_pad, esize;
  int n_slots, ctx_ld, mem_ld;
  int t_rows;                        // rows of the temporal RoPE table
  size_t slot_bytes, slot_v_off, layer_kv_bytes;
  size_t off_kv, off_ctx, ctx_layer_bytes, off_mem, mem_layer_bytes, mem_v_off;
  size_t off_pose, off_sel, off_victim, off_tt, off_th, off_tw, off_w, total;
  bool split;                        // bf16 attention shares key tiles across workgroups
  size_t off_split;                  // split slots: kStreamWG fp32 part states
  bool kf8;                          // FP8 key cache: attention reads E4M3 K with tile exponents
  bool slot8;                        //   held in the slots (K rotated once, at append); else
                                     //   slots keep bf16 raw K and the context buffer is FP8
  size_t slot_kx_off;                // byte offset of the exponents [H][Tpad/64] inside a slot
  int ctx_xtiles;                    // FP8 context buffer: exponents [H][ctx_xtiles] per layer
  size_t ctx_x_off;                  //   at this byte offset inside the layer's buffer
  size_t off_q;                      // bf16: q scratch [T][H][D] of the fused projection path
  int ref_tok, ref_pad;              // reference frames: tokens, padded to whole key tiles
  size_t ref_bytes, ref_v_off, ref_kx_off, off_ref, off_tref;   // per layer, slot-shaped
  bool vf8;                          // FP8 KV cache: attention reads E4M3 V^T with tile exponents
  size_t slot_v8_off, slot_vx_off;   //   inside a slot: E4M3 V^T [H][D][Tpad], exponents [H][Tpad/64]
                                     //   (ConvKV also keeps the raw bf16 V^T at slot_v_off for the conv)
  size_t ref_vx_off;                 //   reference region: E4M3 V^T at ref_v_off, exponents here
  size_t mem_v8_off, mem_vx_off;     //   ConvKV memory: E4M3 V^T [H][D][mem_ld], exponents [H][mem_ld/64]
};

bkv_status validate(const bkv_config* c) {
  if (!c) return fail(BKV_ERR_ARG, "null config");
  if (c->struct_size != sizeof(bkv_config))
    return fail(BKV_ERR_ARG, "config struct_size %u != %zu", c->struct_size, sizeof(bkv_config));
  if (c->mode != BKV_PR_SINK && c->mode != BKV_CONVKV) return fail(BKV_ERR_ARG, "bad mode %d", c->mode);
  if (c->dtype != BKV_F32 && c->dtype != BKV_BF16 && c->dtype != BKV_BF16_FP8K && c->dtype != BKV_BF16_FP8KV)
    return fail(BKV_ERR_ARG, "bad dtype %d", c->dtype);
  if (c->layers < 1 || c->heads < 1) return fail(BKV_ERR_ARG, "layers and heads must be >= 1");
  if (c->rope_positions != BKV_POS_DEFAULT && c->rope_positions != BKV_POS_CONTEXT &&
      c->rope_positions != BKV_POS_ABSOLUTE)
    return fail(BKV_ERR_ARG, "bad rope_positions %d", c->rope_positions);
  if (c->dtype != BKV_F32 && c->head_dim != 128)
    return fail(BKV_ERR_UNSUPPORTED, "bf16 path supports head_dim 128 (got %d)", c->head_dim);
  if (c->dtype == BKV_F32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(BKV_ERR_UNSUPPORTED, "fp32 path supports head_dim 64 or 128 (got %d)", c->head_dim);
  if (c->frames_per_block < 1 || c->grid_h < 1 || c->grid_w < 1)
    return fail(BKV_ERR_ARG, "frames_per_block, grid_h, grid_w must be >= 1");
  const long long T = (long long)c->frames_per_block * c->grid_h * c->grid_w;
  if (T > (1 << 20)) return fail(BKV_ERR_ARG, "block of %lld tokens is too large", T);
  if (c->window_blocks < 1 || c->window_blocks > 8) return fail(BKV_ERR_ARG, "window_blocks must be 1..8");
  const int rs = c->rope_t + c->rope_h + c->rope_w;
  if (c->rope_t < 0 || c->rope_h < 0 || c->rope_w < 0 || (c->rope_t | c->rope_h | c->rope_w) & 1 ||
      (rs != 0 && rs != c->head_dim))
    return fail(BKV_ERR_ARG, "RoPE split must be even parts summing to head_dim (or all 0)");
  if (rs != 0 && !(c->rope_theta > 0.0)) return fail(BKV_ERR_ARG, "rope_theta must be > 0");
  if (c->softmax_scale < 0.f || !std::isfinite(c->softmax_scale))
    return fail(BKV_ERR_ARG, "softmax_scale must be finite and >= 0");
  if (c->mode == BKV_PR_SINK) {
    if (c->static_blocks < 0 || c->static_blocks > 1) return fail(BKV_ERR_ARG, "static_blocks must be 0 or 1");
    if (c->dynamic_k < 0 || c->dynamic_k > bkv::kMaxK) return fail(BKV_ERR_ARG, "dynamic_k must be 0..%d", bkv::kMaxK);
    if (c->bank_blocks < 0 || c->bank_blocks > bkv::kMaxBank)
      return fail(BKV_ERR_ARG, "bank_blocks must be 0..%d", bkv::kMaxBank);
    if (c->dynamic_k > 0 && (c->pose_dim < 1 || c->pose_dim > 1024))
      return fail(BKV_ERR_ARG, "pose_dim must be 1..1024 when dynamic_k > 0");
    if (c->pose_dim < 0) return fail(BKV_ERR_ARG, "pose_dim must be >= 0");
    if (c->reference_frames < 0 || c->reference_frames > 8)
      return fail(BKV_ERR_ARG, "reference_frames must be 0..8");
    if (c->bank_policy != BKV_BANK_FIFO && c->bank_policy != BKV_BANK_POSE)
      return fail(BKV_ERR_ARG, "bad bank_policy %d", c->bank_policy);
    if (c->bank_policy == BKV_BANK_POSE && (c->pose_dim < 1 || c->bank_blocks < 1))
      return fail(BKV_ERR_ARG, "pose-aware bank replacement needs pose_dim >= 1 and bank_blocks >= 1");
    if ((c->reference_frames > 0) + c->static_blocks + c->dynamic_k + c->window_blocks + 1 > bkv::kMaxSeg)
      return fail(BKV_ERR_ARG, "more than %d context segments", bkv::kMaxSeg);
  } else {
    if (c->reference_frames != 0) return fail(BKV_ERR_UNSUPPORTED, "reference frames are implemented for PR-Sink only");
    if (c->bank_policy != BKV_BANK_FIFO) return fail(BKV_ERR_ARG, "ConvKV has no bank");
    if (c->static_blocks != 0 || c->dynamic_k != 0 || c->bank_blocks != 0)
      return fail(BKV_ERR_ARG, "ConvKV takes no static/dynamic sinks or bank");
    if (c->conv_kernel < 1 || c->conv_kernel > 8 || c->conv_stride != c->conv_kernel)
      return fail(BKV_ERR_UNSUPPORTED, "ConvKV needs conv_stride == conv_kernel in 1..8");
    if (c->memory_frames < 1 || c->memory_frames > 4) return fail(BKV_ERR_ARG, "memory_frames must be 1..4");
    if (c->conv_kernel * c->memory_frames > bkv::kMaxTaps) return fail(BKV_ERR_ARG, "too many conv taps");
  }
  return BKV_OK;
}

bkv::Schedule::Shape shape_of(const bkv_config* c) {
  bkv::Schedule::Shape s;
  s.convkv = c->mode == BKV_CONVKV;
  s.layers = c->layers;
  s.frames = c->frames_per_block;
  s.tokens_per_frame = c->grid_h * c->grid_w;
  s.window = c->window_blocks;
  s.statics = s.convkv ? 0 : c->static_blocks;
  s.k = s.convkv ? 0 : c->dynamic_k;
  s.bank = s.convkv ? 0 : c->bank_blocks;
  s.kernel = s.convkv ? c->conv_kernel : 1;
  s.memory_frames = s.convkv ? c->memory_frames : 0;
  s.ref_frames = s.convkv ? 0 : c->reference_frames;
  s.relative = !s.convkv && c->rope_positions == BKV_POS_CONTEXT;
  s.spare = (!s.convkv && c->bank_policy == BKV_BANK_POSE) ? kPoseSpare : 0;
  return s;
}

Layout layout_of(const bkv_config* c, const bkv::Schedule& sch) {
  Layout L{};
  const size_t H = c->heads, D = c->head_dim;
  L.esize = c->dtype == BKV_F32 ? 4 : 2;
  L.kf8 = c->dtype == BKV_BF16_FP8K || c->dtype == BKV_BF16_FP8KV;
  L.vf8 = c->dtype == BKV_BF16_FP8KV;
  L.slot8 = L.kf8 && !sch.ctx_mode();
  const size_t vx_bytes = sizeof(int) * H * (align_up(sch.tokens(), bkv::kTokAlign) / bkv::kTokAlign);
  L.T = sch.tokens();
  L.Tpad = (int)align_up(L.T, bkv::kTokAlign);
  L.Tf = c->grid_h * c->grid_w;
  L.tf_pad = (int)align_up(L.Tf, bkv::kTokAlign);
  L.n_slots = sch.n_slots();
  if (L.slot8 && L.vf8) {
    // [E4M3 K rows H x Tpad x D][K exponents H x Tpad/64][E4M3 V^T H x D x Tpad][V exponents]
    L.slot_kx_off = H * L.Tpad * D;
    L.slot_v_off = L.slot_v8_off = align_up(L.slot_kx_off + vx_bytes, 256);
    L.slot_vx_off = L.slot_v8_off + H * L.Tpad * D;
    L.slot_bytes = align_up(L.slot_vx_off + vx_bytes, 256);
  } else if (L.slot8) {
    // [E4M3 K rows H x Tpad x D][int32 exponents H x Tpad/64][bf16 V^T H x D x Tpad]
    L.slot_kx_off = H * L.Tpad * D;
    L.slot_v_off = align_up(L.slot_kx_off + vx_bytes, 256);
    L.slot_bytes = L.slot_v_off + H * L.Tpad * D * 2;
  } else if (L.vf8) {
    // context modes: [raw bf16 K][raw bf16 V^T, ConvKV only (the conv reads it)][E4M3 V^T][V exponents]
    L.slot_v_off = H * L.Tpad * D * 2;
    L.slot_v8_off = L.slot_v_off + (c->mode == BKV_CONVKV ? H * L.Tpad * D * 2 : 0);
    L.slot_vx_off = L.slot_v8_off + H * L.Tpad * D;
    L.slot_bytes = align_up(L.slot_vx_off + vx_bytes, 256);
  } else {
    L.slot_v_off = H * L.Tpad * D * L.esize;
    L.slot_bytes = 2 * L.slot_v_off;
  }
  L.layer_kv_bytes = L.slot_bytes * L.n_slots;
  // reference frames: one slot-shaped region per layer holding ref_pad tokens
  L.ref_tok = sch.ref_tokens();
  L.ref_pad = (int)align_up(L.ref_tok, bkv::kTokAlign);
  if (L.kf8) {
    L.ref_kx_off = H * L.ref_pad * D;
    L.ref_v_off = align_up(L.ref_kx_off + sizeof(int) * H * (L.ref_pad / bkv::kTokAlign), 256);
    L.ref_vx_off = L.ref_v_off + H * L.ref_pad * D * (L.vf8 ? 1 : 2);
    L.ref_bytes = align_up(L.ref_vx_off + (L.vf8 ? sizeof(int) * H * (L.ref_pad / bkv::kTokAlign) : 0), 256);
  } else {
    L.ref_v_off = align_up(H * L.ref_pad * D * L.esize, 256);
    L.ref_bytes = align_up(L.ref_v_off + H * L.ref_pad * D * L.esize, 256);
  }
  size_t off = 0;
  L.off_kv = off;
  off = align_up(off + L.layer_kv_bytes * c->layers, 256);
  L.off_ref = off;
  if (L.ref_tok > 0) off = align_up(off + L.ref_bytes * c->layers, 256);
  L.off_ctx = off;
  L.off_mem = off;
  if (sch.ctx_mode()) {
    // + one tile: the last segment's partial tile reads up to 63 rows past its end
    L.ctx_ld = (int)align_up(sch.ctx_tokens(), bkv::kTokAlign) + bkv::kTokAlign;
    L.ctx_xtiles = sch.ctx_xtiles();
    L.ctx_x_off = align_up(H * L.ctx_ld * D * (L.kf8 ? 1 : L.esize), 256);
    L.ctx_layer_bytes = align_up(L.ctx_x_off + (L.kf8 ? sizeof(int) * H * L.ctx_xtiles : 0), 256);
    off = align_up(off + L.ctx_layer_bytes * c->layers, 256);
    L.off_mem = off;
  }
  if (c->mode == BKV_CONVKV) {
    L.mem_ld = L.tf_pad * c->memory_frames;
    L.mem_v_off = H * L.mem_ld * D * L.esize;
    L.mem_v8_off = align_up(2 * L.mem_v_off, 256);
    L.mem_vx_off = L.mem_v8_off + H * L.mem_ld * D;
    L.mem_layer_bytes = align_up(L.vf8 ? L.mem_vx_off + sizeof(int) * H * (L.mem_ld / bkv::kTokAlign)
                                       : 2 * L.mem_v_off, 256);
    off = align_up(off + L.mem_layer_bytes * c->layers, 256);
  }
  L.off_pose = off;
  const int P = (c->mode == BKV_PR_SINK) ? c->pose_dim : 0;
  off = align_up(off + sizeof(float) * (size_t)L.n_slots * (P > 0 ? P : 1), 256);
  L.off_sel = off;
  off = align_up(off + 2 * sizeof(int) * bkv::kMaxK, 256);
  L.off_victim = off;                // pose-aware replacement: the bank table [ids | slots]
                                     // (kMaxBank each), then kPoseRing (id, slot) readbacks
  if (c->mode == BKV_PR_SINK && c->bank_policy == BKV_BANK_POSE)
    off = align_up(off + sizeof(int) * (2 * bkv::kMaxBank + 2 * kPoseRing), 256);
  L.t_rows = sch.ctx_mode() ? sch.max_context_frames() : c->frames_per_block;
  L.off_tt = off;
  off = align_up(off + sizeof(float2) * (size_t)L.t_rows * (c->rope_t / 2 + 1), 256);
  L.off_tref = off;
  if (L.ref_tok > 0) off = align_up(off + sizeof(float2) * (size_t)c->reference_frames * (c->rope_t / 2 + 1), 256);
  L.off_th = off;
  off = align_up(off + sizeof(float2) * (size_t)c->grid_h * (c->rope_h / 2 + 1), 256);
  L.off_tw = off;
  off = align_up(off + sizeof(float2) * (size_t)c->grid_w * (c->rope_w / 2 + 1), 256);
  L.off_w = off;
  if (c->mode == BKV_CONVKV) off = align_up(off + sizeof(float) * 2 * c->layers * H * D * c->conv_kernel, 256);
  const long long units = (long long)H * ((L.T + bkv::kAttnBM - 1) / bkv::kAttnBM);
  L.split = c->dtype != BKV_F32 && units > bkv::kStreamWG;
  L.off_split = off;
  if (L.split) off = align_up(off + bkv::kSplitSlotBytes * bkv::kStreamWG, 256);
  L.off_q = off;
  if (c->dtype != BKV_F32) off = align_up(off + (size_t)L.T * H * D * 2, 256);
  L.total = off;
  return L;
}

}  // namespace

struct bkv_cache_s {
  bkv_config cfg;
  bkv::Schedule sched;
  Layout L;
  char* ws;
  int device;
  bool error = false;
  std::vector<bool> ctx_ready;      // ConvKV: context K of the layer gathered for the open block
  std::vector<bool> weights_set;    // ConvKV: conv weights given per layer
  std::vector<bool> ref_set;        // PR-Sink: reference frames given per layer
  int64_t split_attends = 0;        // bf16 attention launches that used the split launch
  // pose-aware bank: displaced (id, slot) pairs read back into pinned host
  // memory, each with an event recorded after its copy; ring positions in
  // flight, oldest first
  int* victim_host = nullptr;
  hipEvent_t victim_ev[kPoseRing] = {};
  std::vector<int> victim_pending;
  int victim_next = 0;
  struct Prof {                     // per-launch HIP event pairs (bkv_profile_start/stop)
    bool on = false;
    int cap = 0, used = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> tag;
  } prof;

  bkv_cache_s(const bkv_config& c, char* w)
      : cfg(c), sched(shape_of(&c)), ws(w), device(0) {
    L = layout_of(&c, sched);
    ctx_ready.assign(c.layers, false);
    weights_set.assign(c.layers, false);
    ref_set.assign(c.layers, false);
  }

  bool bf16() const { return cfg.dtype != BKV_F32; }   // bf16 Q/K/V/out and V cache
  bool kf8() const { return L.kf8; }
  bool slot8() const { return L.slot8; }
  bool convkv() const { return cfg.mode == BKV_CONVKV; }
  // ConvKV or context-relative PR-Sink: slots hold raw K; the context's K is
  // rotated per block into the context-K buffer at context positions.
  bool ctx_mode() const { return sched.ctx_mode(); }
  // ConvKV with only the memory's positions restarted: the t-table rows keep
  // the context-relative layout, their values are rewritten every block.
  bool conv_abs() const { return convkv() && cfg.rope_positions == BKV_POS_ABSOLUTE; }
  char* layer_kv(int l) const { return ws + L.off_kv + L.layer_kv_bytes * l; }
  char* slot_k(int l, int s) const { return layer_kv(l) + L.slot_bytes * s; }
  char* slot_vt(int l, int s) const { return slot_k(l, s) + L.slot_v_off; }
  bool vf8() const { return L.vf8; }
  char* slot_v8(int l, int s) const { return slot_k(l, s) + L.slot_v8_off; }
  int* slot_vx(int l, int s) const { return reinterpret_cast<int*>(slot_k(l, s) + L.slot_vx_off); }
  // the V^T that attention reads: E4M3 with the FP8 KV cache, else bf16
  size_t slot_va_off() const { return L.vf8 ? L.slot_v8_off : L.slot_v_off; }
  int* slot_kx(int l, int s) const { return reinterpret_cast<int*>(slot_k(l, s) + L.slot_kx_off); }
  long long slot_kx_hs() const { return L.Tpad / bkv::kTokAlign; }
  char* ctx_k(int l) const { return ws + L.off_ctx + L.ctx_layer_bytes * l; }
  int* ctx_x(int l) const { return reinterpret_cast<int*>(ctx_k(l) + L.ctx_x_off); }
  size_t ctx_esize() const { return kf8() ? 1 : L.esize; }   // bytes per context K value
  // context-buffer view of a segment's K (rows from ctx_off; FP8: its exponents)
  void ctx_seg_k(int l, const bkv::SegPlan& p, bkv::Seg& g) const {
    g.k = ctx_k(l) + (size_t)p.ctx_off * cfg.head_dim * ctx_esize();
    g.k_hs = (long long)L.ctx_ld * cfg.head_dim;
    if (kf8()) {
      g.kx = ctx_x(l) + p.x_off;
      g.kx_hs = L.ctx_xtiles;
    }
  }
  char* mem_k(int l) const { return ws + L.off_mem + L.mem_layer_bytes * l; }
  char* mem_vt(int l) const { return mem_k(l) + L.mem_v_off; }
  char* mem_v8(int l) const { return mem_k(l) + L.mem_v8_off; }
  int* mem_vx(int l) const { return reinterpret_cast<int*>(mem_k(l) + L.mem_vx_off); }
  float* pose_store() const { return reinterpret_cast<float*>(ws + L.off_pose); }
  int* sel_ids() const { return reinterpret_cast<int*>(ws + L.off_sel); }
  int* sel_slots() const { return sel_ids() + bkv::kMaxK; }
  float2* ttab() const { return reinterpret_cast<float2*>(ws + L.off_tt); }
  float2* htab() const { return reinterpret_cast<float2*>(ws + L.off_th); }
  float2* wtab() const { return reinterpret_cast<float2*>(ws + L.off_tw); }
  float* conv_w(int l, int which) const {
    const size_t n = (size_t)cfg.heads * cfg.head_dim * cfg.conv_kernel;
    return reinterpret_cast<float*>(ws + L.off_w) + (2 * (size_t)l + which) * n;
  }
  bool pose_bank() const { return cfg.mode == BKV_PR_SINK && cfg.bank_policy == BKV_BANK_POSE; }
  int* bank_dev() const { return reinterpret_cast<int*>(ws + L.off_victim); }
  int* victim_dev(int r) const { return bank_dev() + 2 * bkv::kMaxBank + 2 * r; }
  char* ref_k(int l) const { return ws + L.off_ref + L.ref_bytes * l; }
  char* ref_vt(int l) const { return ref_k(l) + L.ref_v_off; }
  int* ref_vx(int l) const { return reinterpret_cast<int*>(ref_k(l) + L.ref_vx_off); }
  int* ref_kx(int l) const { return reinterpret_cast<int*>(ref_k(l) + L.ref_kx_off); }
  float2* tref() const { return reinterpret_cast<float2*>(ws + L.off_tref); }
  long long slot_k_hs() const { return (long long)L.Tpad * cfg.head_dim; }
  long long slot_v_hs() const { return (long long)L.Tpad * cfg.head_dim; }

  bkv::Rope rope() const {
    bkv::Rope r;
    r.t = ttab();
    r.h = htab();
    r.w = wtab();
    r.dt = cfg.rope_t;
    r.dh = cfg.rope_h;
    r.dw = cfg.rope_w;
    r.grid_h = cfg.grid_h;
    r.grid_w = cfg.grid_w;
    return r;
  }

  // attention view of context segment i of the open block at layer l
  bkv::Seg seg_arg(int l, const bkv::SegPlan& p) const {
    bkv::Seg g{};
    g.n = p.tokens;
    g.dyn = p.dyn;
    if (p.dyn >= 0) {                 // slot known on device; K from the context buffer if rotated there
      if (ctx_mode()) ctx_seg_k(l, p, g);
      return g;
    }
    if (p.kind == bkv::SEG_REFERENCE) {
      g.k = ref_k(l);
      g.v = ref_vt(l);
      g.k_hs = g.v_hs = (long long)L.ref_pad * cfg.head_dim;
      g.v_ld = L.ref_pad;
      if (kf8()) {
        g.kx = ref_kx(l);
        g.kx_hs = L.ref_pad / bkv::kTokAlign;
      }
      if (vf8()) {
        g.vx = ref_vx(l);
        g.vx_hs = L.ref_pad / bkv::kTokAlign;
      }
    } else if (!ctx_mode()) {
      g.k = slot_k(l, p.slot);
      g.v = slot_k(l, p.slot) + slot_va_off();
      g.k_hs = slot_k_hs();
      g.v_hs = slot_v_hs();
      g.v_ld = L.Tpad;
      if (slot8()) {
        g.kx = slot_kx(l, p.slot);
        g.kx_hs = slot_kx_hs();
      }
      if (vf8()) {
        g.vx = slot_vx(l, p.slot);
        g.vx_hs = slot_kx_hs();
      }
    } else {
      ctx_seg_k(l, p, g);
      if (p.kind == bkv::SEG_MEMORY) {
        const size_t col = (size_t)p.id * L.tf_pad;       // the frame's first V^T column
        g.v = vf8() ? mem_v8(l) + col : mem_vt(l) + col * L.esize;
        g.v_hs = (long long)L.mem_ld * cfg.head_dim;
        g.v_ld = L.mem_ld;
        if (vf8()) {
          g.vx = mem_vx(l) + col / bkv::kTokAlign;
          g.vx_hs = L.mem_ld / bkv::kTokAlign;
        }
      } else {
        g.v = slot_k(l, p.slot) + slot_va_off();
        g.v_hs = slot_v_hs();
        g.v_ld = L.Tpad;
        if (vf8()) {
          g.vx = slot_vx(l, p.slot);
          g.vx_hs = slot_kx_hs();
        }
      }
    }
    return g;
  }
};

namespace {

void profile_release(bkv_cache h) {
  for (hipEvent_t e : h->prof.ev)
    if (e) (void)hipEventDestroy(e);
  h->prof = bkv_cache_s::Prof{};
}

// Pose-aware bank: wait for every displaced-member readback in flight and
// forget them (reset, destroy).
void victims_drain(bkv_cache h) {
  for (int r : h->victim_pending) (void)hipEventSynchronize(h->victim_ev[r]);
  h->victim_pending.clear();
}

void victims_release(bkv_cache h) {
  victims_drain(h);
  for (hipEvent_t& e : h->victim_ev)
    if (e) {
      (void)hipEventDestroy(e);
      e = nullptr;
    }
  if (h->victim_host) (void)hipHostFree(h->victim_host);
  h->victim_host = nullptr;
}

bkv_status check_handle(bkv_cache h, bool need_ok = true) {
  if (!h) return fail(BKV_ERR_ARG, "null handle");
  if (need_ok && h->error) return fail(BKV_ERR_STATE, "handle is in error state; call bkv_reset");
  return BKV_OK;
}

enum { K_RETRIEVE = 0, K_APPEND, K_ATTENTION, K_GATHER, K_CONV, K_EXPORT, K_QKV, K_REPLACE, K_VQUANT, K_COUNT };
const char* const kKernelNames[K_COUNT] = {"retrieve", "append", "attention", "gather", "conv", "export",
                                           "qkv", "replace", "vquant"};

// Run `launch`, bracketed by event records on `s` while a profile is recording.
template <class F>
hipError_t timed(bkv_cache h, int tag, hipStream_t s, F&& launch) {
  auto& p = h->prof;
  const bool rec = p.on && p.used < p.cap;
  if (rec) (void)hipEventRecord(p.ev[2 * p.used], s);
  hipError_t e = launch();
  if (rec) {
    (void)hipEventRecord(p.ev[2 * p.used + 1], s);
    p.tag[p.used++] = tag;
  }
  return e;
}

bkv_status device_fail(bkv_cache h, hipError_t e, const char* what) {
  h->error = true;
  return fail(BKV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bkv_status set_device(bkv_cache h) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_fail(h, e, "hipGetDevice");
  if (cur != h->device) {
    e = hipSetDevice(h->device);
    if (e != hipSuccess) return device_fail(h, e, "hipSetDevice");
  }
  return BKV_OK;
}

// ConvKV / context-relative PR-Sink: rotate the raw K of the context's cached
// segments (memory frames; static, retrieved and window blocks) of layer l
// into the context-K buffer at their context positions.
bkv_status gather_context(bkv_cache h, int l, hipStream_t stream) {
  bkv::GatherArgs g{};
  g.dst = h->ctx_k(l);
  g.dst_hs = (long long)h->L.ctx_ld * h->cfg.head_dim;
  g.kf8 = h->kf8() ? 1 : 0;
  g.dx = h->kf8() ? h->ctx_x(l) : nullptr;
  g.dx_hs = h->L.ctx_xtiles;
  g.H = h->cfg.heads;
  g.D = h->cfg.head_dim;
  g.rope = h->rope();
  g.sel_ids = h->sel_ids();
  g.sel_slots = h->sel_slots();
  g.slot_base = h->layer_kv(l);
  g.slot_bytes = (long long)h->L.slot_bytes;
  g.slot_k_hs = h->slot_k_hs();
  g.n_dyn = h->sched.n_dynamic();
  g.frames = h->cfg.frames_per_block;
  for (const auto& p : h->sched.segments()) {
    if (p.kind == bkv::SEG_CURRENT || p.kind == bkv::SEG_REFERENCE) continue;
    bkv::GatherPart& gp = g.part[g.nparts++];
    gp.dyn = p.dyn;
    if (p.dyn >= 0) {
      gp.src = nullptr;                 // the selected slot, on device
      gp.src_hs = 0;
    } else if (p.kind == bkv::SEG_MEMORY) {
      gp.src = h->mem_k(l) + (size_t)p.id * h->L.tf_pad * h->cfg.head_dim * h->L.esize;
      gp.src_hs = (long long)h->L.mem_ld * h->cfg.head_dim;
    } else {
      gp.src = h->slot_k(l, p.slot);
      gp.src_hs = h->slot_k_hs();
    }
    gp.dst_off = p.ctx_off;
    gp.x_off = p.x_off;
    gp.n = p.tokens;
    gp.t_row0 = (int)p.t0;
    if (gp.n > g.max_n) g.max_n = gp.n;
  }
  hipError_t e = timed(h, K_GATHER, stream, [&] { return bkv::launch_gather(g, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "gather launch");
  h->ctx_ready[l] = true;
  return BKV_OK;
}

}  // namespace

extern "C" {

const char* bkv_status_str(bkv_status s) {
  switch (s) {
    case BKV_OK: return "BKV_OK";
    case BKV_ERR_ARG: return "BKV_ERR_ARG";
    case BKV_ERR_STATE: return "BKV_ERR_STATE";
    case BKV_ERR_WORKSPACE: return "BKV_ERR_WORKSPACE";
    case BKV_ERR_DEVICE: return "BKV_ERR_DEVICE";
    case BKV_ERR_UNSUPPORTED: return "BKV_ERR_UNSUPPORTED";
  }
  return "BKV_ERR_UNKNOWN";
}

const char* bkv_last_error(void) { return g_err.c_str(); }

bkv_status bkv_workspace_size(const bkv_config* cfg, size_t* bytes) {
  if (!bytes) return fail(BKV_ERR_ARG, "null bytes");
  bkv_status st = validate(cfg);
  if (st != BKV_OK) return st;
  bkv::Schedule sch(shape_of(cfg));
  *bytes = layout_of(cfg, sch).total;
  return BKV_OK;
}

bkv_status bkv_create(const bkv_config* cfg, void* workspace, size_t bytes, hipStream_t stream,
                      bkv_cache* out) {
  if (!out) return fail(BKV_ERR_ARG, "null out");
  *out = nullptr;
  bkv_status st = validate(cfg);
  if (st != BKV_OK) return st;
  size_t need = 0;
  bkv_workspace_size(cfg, &need);
  if (!workspace) return fail(BKV_ERR_WORKSPACE, "null workspace");
  if (bytes < need) return fail(BKV_ERR_WORKSPACE, "workspace %zu < needed %zu bytes", bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(BKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  bkv_cache h = new (std::nothrow) bkv_cache_s(*cfg, static_cast<char*>(workspace));
  if (!h) return fail(BKV_ERR_ARG, "out of host memory");
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return fail(BKV_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  }
  // Zero once: attention tiles read the pad columns of V^T buffers (never
  // written afterwards) and must see finite values there.
  e = hipMemsetAsync(workspace, 0, need, stream);
  if (e != hipSuccess) {
    delete h;
    return fail(BKV_ERR_DEVICE, "workspace clear: %s", hipGetErrorString(e));
  }
  const double theta = cfg->rope_theta;
  if (cfg->rope_h) e = bkv::launch_rope_table(h->htab(), cfg->grid_h, cfg->rope_h, 0, theta, stream);
  if (e == hipSuccess && cfg->rope_w)
    e = bkv::launch_rope_table(h->wtab(), cfg->grid_w, cfg->rope_w, 0, theta, stream);
  if (e == hipSuccess && cfg->rope_t && h->ctx_mode() && !h->conv_abs())
    e = bkv::launch_rope_table(h->ttab(), h->L.t_rows, cfg->rope_t, 0, theta, stream);
  if (e == hipSuccess && cfg->rope_t && h->L.ref_tok > 0)
    e = bkv::launch_rope_table(h->tref(), cfg->reference_frames, cfg->rope_t, 0, theta, stream);
  if (e != hipSuccess) {
    delete h;
    return fail(BKV_ERR_DEVICE, "RoPE table launch: %s", hipGetErrorString(e));
  }
  if (h->pose_bank()) {               // pinned host words for the displaced-member readbacks
    e = hipHostMalloc(reinterpret_cast<void**>(&h->victim_host), sizeof(int) * 2 * kPoseRing);
    for (int r = 0; r < kPoseRing && e == hipSuccess; ++r)
      e = hipEventCreateWithFlags(&h->victim_ev[r], hipEventDisableTiming);
    if (e != hipSuccess) {
      victims_release(h);
      delete h;
      return fail(BKV_ERR_DEVICE, "pose bank readback set-up: %s", hipGetErrorString(e));
    }
  }
  *out = h;
  return BKV_OK;
}

bkv_status bkv_destroy(bkv_cache h) {
  if (!h) return fail(BKV_ERR_ARG, "null handle");
  profile_release(h);
  victims_release(h);
  delete h;
  return BKV_OK;
}

bkv_status bkv_reset(bkv_cache h) {
  if (!h) return fail(BKV_ERR_ARG, "null handle");
  victims_drain(h);
  h->sched.reset();
  h->error = false;
  h->ctx_ready.assign(h->cfg.layers, false);
  h->split_attends = 0;
  return BKV_OK;
}

bkv_status bkv_set_conv_weights(bkv_cache h, int32_t layer, const float* wk, const float* wv,
                                hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (!h->convkv()) return fail(BKV_ERR_UNSUPPORTED, "conv weights on a PR-Sink handle");
  if (layer < 0 || layer >= h->cfg.layers) return fail(BKV_ERR_ARG, "layer %d out of range", layer);
  if (!wk || !wv) return fail(BKV_ERR_ARG, "null weights");
  if ((st = set_device(h)) != BKV_OK) return st;
  const size_t n = sizeof(float) * h->cfg.heads * h->cfg.head_dim * h->cfg.conv_kernel;
  hipError_t e = hipMemcpyAsync(h->conv_w(layer, 0), wk, n, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(h->conv_w(layer, 1), wv, n, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return device_fail(h, e, "conv weight copy");
  h->weights_set[layer] = true;
  return BKV_OK;
}

bkv_status bkv_set_reference(bkv_cache h, int32_t layer, const void* k, const void* v, hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (h->L.ref_tok == 0) return fail(BKV_ERR_UNSUPPORTED, "the handle has no reference frames");
  if (h->sched.is_open()) return fail(BKV_ERR_STATE, "reference set while block %lld is open",
                                      (long long)h->sched.block());
  if (layer < 0 || layer >= h->cfg.layers) return fail(BKV_ERR_ARG, "layer %d out of range", layer);
  if (!k || !v) return fail(BKV_ERR_ARG, "null k or v");
  if (k == v) return fail(BKV_ERR_ARG, "k aliases v");
  if ((st = set_device(h)) != BKV_OK) return st;
  bkv::AppendArgs ap{};
  ap.k_in = k;
  ap.v_in = v;
  ap.T = h->L.ref_tok;
  ap.H = h->cfg.heads;
  ap.D = h->cfg.head_dim;
  ap.rope = h->rope();
  ap.rope.t = h->tref();              // frame f of the reference at t = f
  ap.t_row0 = 0;
  ap.vt = h->ref_vt(layer);
  ap.vt_hs = (long long)h->L.ref_pad * h->cfg.head_dim;
  ap.vt_ld = h->L.ref_pad;
  if (h->vf8()) {
    ap.v8 = ap.vt;
    ap.v8_hs = ap.vt_hs;
    ap.v8_ld = ap.vt_ld;
    ap.vt = nullptr;
    ap.vx = h->ref_vx(layer);
    ap.vx_hs = h->L.ref_pad / bkv::kTokAlign;
  }
  if (h->kf8()) {
    ap.k8 = h->ref_k(layer);
    ap.k8_hs = ap.vt_hs;
    ap.kx = h->ref_kx(layer);
    ap.kx_hs = h->L.ref_pad / bkv::kTokAlign;
  } else {
    ap.k_rot = h->ref_k(layer);
    ap.k_rot_hs = ap.vt_hs;
  }
  hipError_t e = timed(h, K_APPEND, stream, [&] { return bkv::launch_append(ap, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "reference append launch");
  h->ref_set[layer] = true;
  return BKV_OK;
}

bkv_status bkv_retrieve(bkv_cache h, const float* pose, hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (h->sched.is_open()) return fail(BKV_ERR_STATE, "block %lld is already open", (long long)h->sched.block());
  const bool prsink = !h->convkv();
  const bool needs_pose = prsink && h->cfg.dynamic_k > 0;
  if (needs_pose && !pose) return fail(BKV_ERR_ARG, "null pose");
  if (h->convkv()) {
    for (int l = 0; l < h->cfg.layers; ++l)
      if (!h->weights_set[l]) return fail(BKV_ERR_STATE, "conv weights of layer %d not set", l);
  }
  if (h->L.ref_tok > 0) {
    for (int l = 0; l < h->cfg.layers; ++l)
      if (!h->ref_set[l]) return fail(BKV_ERR_STATE, "reference frames of layer %d not set", l);
  }
  if ((st = set_device(h)) != BKV_OK) return st;
  // pose-aware bank: take in the displaced members whose readback has
  // landed; wait for the oldest only when no slot is free (the host is then
  // kPoseSpare blocks ahead of the device)
  while (!h->victim_pending.empty()) {
    const int r = h->victim_pending.front();
    hipError_t e = hipEventQuery(h->victim_ev[r]);
    if (e == hipErrorNotReady) {
      if (h->sched.free_slots() > 0) break;
      e = hipEventSynchronize(h->victim_ev[r]);
    }
    if (e != hipSuccess) return device_fail(h, e, "bank replacement readback");
    if (!h->sched.resolve_displaced(h->victim_host[2 * r])) {
      h->error = true;
      return fail(BKV_ERR_DEVICE, "bank replacement returned id %d, not a bank member", h->victim_host[2 * r]);
    }
    h->victim_pending.erase(h->victim_pending.begin());
  }
  if (!h->sched.open()) return fail(BKV_ERR_STATE, "no free slot (internal)");
  h->ctx_ready.assign(h->cfg.layers, false);
  if (h->conv_abs() && h->cfg.rope_t) {
    // rows [0, n_mem): memory frames at 0..n_mem-1; the rows after them: the
    // window's first block onward at absolute frame indices
    const auto& segs = h->sched.segments();
    int n_mem = 0;
    while (n_mem < (int)segs.size() && segs[n_mem].kind == bkv::SEG_MEMORY) ++n_mem;
    const int64_t first = segs[n_mem].id;          // oldest window block, or the current block
    const int rows = (int)(segs.size() - n_mem) * h->cfg.frames_per_block;
    const int half = h->cfg.rope_t / 2;
    hipError_t e = hipSuccess;
    if (n_mem > 0)
      e = timed(h, K_RETRIEVE, stream, [&] {
        return bkv::launch_rope_table(h->ttab(), n_mem, h->cfg.rope_t, 0, h->cfg.rope_theta, stream);
      });
    if (e == hipSuccess)
      e = timed(h, K_RETRIEVE, stream, [&] {
        return bkv::launch_rope_table(h->ttab() + (size_t)n_mem * half, rows, h->cfg.rope_t,
                                      first * h->cfg.frames_per_block, h->cfg.rope_theta, stream);
      });
    if (e != hipSuccess) return device_fail(h, e, "RoPE table launch");
  }
  if (prsink) {
    bkv::OpenArgs a{};
    a.pose_in = needs_pose ? pose : nullptr;
    a.pose_store = h->pose_store();
    a.P = h->cfg.pose_dim;
    a.cur_slot = h->sched.cur_slot();
    a.k = h->sched.n_dynamic();
    a.nbank = a.k > 0 ? h->sched.bank_count() : 0;
    a.upd_pos = -1;
    if (h->pose_bank()) {
      a.bank_dev = h->bank_dev();       // the device holds the pose-aware bank
    } else {
      for (int i = 0; i < a.nbank; ++i) {
        a.bank_id[i] = (int)h->sched.bank()[i].first;
        a.bank_slot[i] = h->sched.bank()[i].second;
      }
    }
    a.sel_ids = h->sel_ids();
    a.sel_slots = h->sel_slots();
    if (h->cfg.rope_t && !h->ctx_mode()) {   // absolute positions: this block's t rows
      a.ttab = h->ttab();
      a.t_rows = h->cfg.frames_per_block;
      a.t_dim = h->cfg.rope_t;
      a.t_pos0 = h->sched.block_t0(h->sched.block());
      a.theta = h->cfg.rope_theta;
    }
    if (a.pose_in || a.ttab || a.k > 0) {
      hipError_t e = timed(h, K_RETRIEVE, stream, [&] { return bkv::launch_open(a, stream); });
      if (e != hipSuccess) return device_fail(h, e, "retrieval launch");
    }
  }
  return BKV_OK;
}

}  // extern "C"

namespace {

// Destinations of the current block's K and V at `layer` (append kernel or
// the fused projection's epilogue).
bkv::AppendArgs append_args(bkv_cache h, int layer) {
  const auto& cur = h->sched.segments().back();
  const int D = h->cfg.head_dim;
  bkv::AppendArgs ap{};
  ap.T = h->L.T;
  ap.H = h->cfg.heads;
  ap.D = D;
  ap.rope = h->rope();
  ap.vt = h->slot_vt(layer, cur.slot);
  ap.vt_hs = h->slot_v_hs();
  ap.vt_ld = h->L.Tpad;
  if (h->vf8()) {                     // E4M3 V^T; the raw bf16 V^T only where the conv reads it
    ap.v8 = h->slot_v8(layer, cur.slot);
    ap.v8_hs = h->slot_v_hs();
    ap.v8_ld = h->L.Tpad;
    ap.vx = h->slot_vx(layer, cur.slot);
    ap.vx_hs = h->slot_kx_hs();
    if (!h->convkv()) ap.vt = nullptr;
  }
  if (h->slot8()) {
    ap.k8 = h->slot_k(layer, cur.slot);
    ap.k8_hs = h->slot_k_hs();
    ap.kx = h->slot_kx(layer, cur.slot);
    ap.kx_hs = h->slot_kx_hs();
    ap.t_row0 = 0;
  } else if (h->kf8()) {              // raw K to the slot, E4M3 K~ into the context buffer
    ap.k_raw = h->slot_k(layer, cur.slot);
    ap.k_raw_hs = h->slot_k_hs();
    ap.k8 = h->ctx_k(layer) + (size_t)cur.ctx_off * D;
    ap.k8_hs = (long long)h->L.ctx_ld * D;
    ap.kx = h->ctx_x(layer) + cur.x_off;
    ap.kx_hs = h->L.ctx_xtiles;
    ap.t_row0 = (int)cur.t0;
  } else if (!h->ctx_mode()) {
    ap.k_rot = h->slot_k(layer, cur.slot);
    ap.k_rot_hs = h->slot_k_hs();
    ap.k_rot_off = 0;
    ap.t_row0 = 0;
  } else {
    ap.k_raw = h->slot_k(layer, cur.slot);
    ap.k_raw_hs = h->slot_k_hs();
    ap.k_rot = h->ctx_k(layer);
    ap.k_rot_hs = (long long)h->L.ctx_ld * D;
    ap.k_rot_off = cur.ctx_off;
    ap.t_row0 = (int)cur.t0;
  }
  return ap;
}

// After the current block's K/V are in the cache: ConvKV context gather (once
// per layer and block), then attention of q over the context into out.
// static_slots: the split launch's part states go to the static device array
// (the allocation-free attend) instead of the workspace's split slots.
bkv_status attend_context(bkv_cache h, int layer, const void* q, void* out, hipStream_t stream,
                          float* static_slots = nullptr) {
  bkv_status st;
  if (h->ctx_mode() && !h->ctx_ready[layer]) {
    if ((st = gather_context(h, layer, stream)) != BKV_OK) return st;
  }
  const auto& segs = h->sched.segments();
  const auto& cur = segs.back();
  const int D = h->cfg.head_dim;
  bkv::AttnArgs a{};
  a.q = q;
  a.out = out;
  a.T = h->L.T;
  a.H = h->cfg.heads;
  a.D = D;
  a.t_row0 = h->ctx_mode() ? (int)cur.t0 : 0;
  const float scale = h->cfg.softmax_scale > 0.f ? h->cfg.softmax_scale : 1.0f / std::sqrt((float)D);
  a.qscale = scale * 1.4426950408889634f;   // base-2 logits on both paths
  a.rope = h->rope();
  a.sel_slots = h->sel_slots();
  a.slot_base = h->layer_kv(layer);
  a.slot_bytes = (long long)h->L.slot_bytes;
  a.slot_v_off = (long long)h->slot_va_off();
  a.slot_k_hs = h->slot_k_hs();
  a.slot_v_hs = h->slot_v_hs();
  a.slot_v_ld = h->L.Tpad;
  a.kf8 = h->kf8() ? 1 : 0;
  a.slot_kx_off = (long long)h->L.slot_kx_off;
  a.slot_kx_hs = h->slot_kx_hs();
  a.vf8 = h->vf8() ? 1 : 0;
  a.slot_vx_off = (long long)h->L.slot_vx_off;
  a.slot_vx_hs = h->slot_kx_hs();
  a.split = h->L.split ? 1 : 0;
  a.part = static_slots ? static_slots : reinterpret_cast<float*>(h->ws + h->L.off_split);
  a.nseg = (int)segs.size();
  for (int i = 0; i < a.nseg; ++i) a.seg[i] = h->seg_arg(layer, segs[i]);
  hipError_t e = timed(h, K_ATTENTION, stream, [&] { return bkv::launch_attention(a, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "attention launch");
  if (h->bf16() && bkv::attention_split(a.T, a.H, a.split != 0)) ++h->split_attends;
  h->sched.mark_attended(layer);
  return BKV_OK;
}

// handle, open block and layer checks shared by the attend calls
bkv_status attend_checks(bkv_cache h, int32_t layer) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (!h->sched.is_open()) return fail(BKV_ERR_STATE, "attend with no open block");
  if (layer < 0 || layer >= h->cfg.layers) return fail(BKV_ERR_ARG, "layer %d out of range", layer);
  return BKV_OK;
}

}  // namespace

extern "C" {

bkv_status bkv_attend(bkv_cache h, int32_t layer, const void* q, const void* k, const void* v,
                      void* out, hipStream_t stream) {
  bkv_status st = attend_checks(h, layer);
  if (st != BKV_OK) return st;
  if (!q || !k || !v || !out) return fail(BKV_ERR_ARG, "null q/k/v/out");
  if (out == q || out == k || out == v) return fail(BKV_ERR_ARG, "out aliases an input");
  if ((st = set_device(h)) != BKV_OK) return st;
  bkv::AppendArgs ap = append_args(h, layer);
  ap.k_in = k;
  ap.v_in = v;
  hipError_t e = timed(h, K_APPEND, stream, [&] { return bkv::launch_append(ap, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "append launch");
  return attend_context(h, layer, q, out, stream);
}

bkv_status bkv_attend_static_scratch(bkv_cache h, int32_t layer, const void* q, const void* k, const void* v,
                                     void* out, hipStream_t stream) {
  bkv_status st = attend_checks(h, layer);
  if (st != BKV_OK) return st;
  if (!q || !k || !v || !out) return fail(BKV_ERR_ARG, "null q/k/v/out");
  if (out == q || out == k || out == v) return fail(BKV_ERR_ARG, "out aliases an input");
  if ((st = set_device(h)) != BKV_OK) return st;
  float* slots = nullptr;
  hipError_t e = bkv::static_split_slots(&slots);
  if (e != hipSuccess) return device_fail(h, e, "static split slots");
  bkv::AppendArgs ap = append_args(h, layer);
  ap.k_in = k;
  ap.v_in = v;
  e = timed(h, K_APPEND, stream, [&] { return bkv::launch_append(ap, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "append launch");
  return attend_context(h, layer, q, out, stream, slots);
}

bkv_status bkv_attend_qkv(bkv_cache h, int32_t layer, const void* x, const void* w, const void* b,
                          int32_t model_dim, void* out, hipStream_t stream) {
  bkv_status st = attend_checks(h, layer);
  if (st != BKV_OK) return st;
  if (h->cfg.dtype == BKV_F32)
    return fail(BKV_ERR_UNSUPPORTED, "the fused QKV projection is implemented for the bf16 cache dtypes");
  if (!x || !w || !out) return fail(BKV_ERR_ARG, "null x, w or out");
  if (out == x || out == w || out == b) return fail(BKV_ERR_ARG, "out aliases an input");
  if (model_dim <= 0 || model_dim % 32 != 0) return fail(BKV_ERR_ARG, "model_dim must be a positive multiple of 32");
  const long long rows = 3LL * h->cfg.heads * h->cfg.head_dim;
  if ((long long)h->L.T * model_dim * 2 >= (1LL << 31) || rows * model_dim * 2 >= (1LL << 31))
    return fail(BKV_ERR_UNSUPPORTED, "x or w exceeds 2 GiB");
  if ((st = set_device(h)) != BKV_OK) return st;
  bkv::QkvArgs g{};
  g.x = x;
  g.w = w;
  g.b = b;
  g.C = model_dim;
  g.q = h->ws + h->L.off_q;
  g.ap = append_args(h, layer);
  hipError_t e = timed(h, K_QKV, stream, [&] { return bkv::launch_qkv(g, stream); });
  if (e != hipSuccess) return device_fail(h, e, "qkv projection launch");
  return attend_context(h, layer, g.q, out, stream);
}

bkv_status bkv_commit(bkv_cache h, hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (!h->sched.is_open()) return fail(BKV_ERR_STATE, "commit with no open block");
  if (!h->sched.all_attended()) return fail(BKV_ERR_STATE, "commit before every layer was attended");
  if ((st = set_device(h)) != BKV_OK) return st;
  int displace = -1;
  if (h->pose_bank()) {
    const auto ev = h->sched.pending_eviction();
    if (ev.first >= 0) {
      // The leaving block joins the device's bank table: at the next free
      // position while there is room; in a full bank it replaces the member
      // ranked first against its stored pose (top 1), whose (id, slot) are
      // copied back to pinned host memory and taken in by a later retrieve.
      // Nothing here waits for the device.
      const bool full = h->sched.bank_full();
      if (full && (int)h->victim_pending.size() >= kPoseRing)
        return fail(BKV_ERR_STATE, "too many bank replacements in flight (internal)");
      bkv::OpenArgs a{};
      a.pose_store = h->pose_store();
      a.P = h->cfg.pose_dim;
      a.cur_slot = -1;
      a.bank_dev = h->bank_dev();
      a.upd_id = (int)ev.first;
      a.upd_slot = ev.second;
      a.upd_pos = full ? -1 : h->sched.bank_count();
      const int r = h->victim_next;
      if (full) {
        a.query = h->pose_store() + (size_t)ev.second * h->cfg.pose_dim;
        a.k = 1;
        a.nbank = h->sched.bank_count();
        a.victim_out = h->victim_dev(r);
        a.sel_ids = h->victim_dev(r);  // the ranking's own outputs land in the same pair
        a.sel_slots = h->victim_dev(r) + 1;
      }
      hipError_t e = timed(h, K_REPLACE, stream, [&] { return bkv::launch_open(a, stream); });
      if (e == hipSuccess && full)
        e = hipMemcpyAsync(h->victim_host + 2 * r, h->victim_dev(r), 2 * sizeof(int), hipMemcpyDeviceToHost,
                           stream);
      if (e == hipSuccess && full) e = hipEventRecord(h->victim_ev[r], stream);
      if (e != hipSuccess) return device_fail(h, e, "bank replacement");
      if (full) {
        h->victim_pending.push_back(r);
        h->victim_next = (r + 1) % kPoseRing;
        displace = bkv::Schedule::kDisplaceDeferred;
      }
    }
  }
  std::vector<bkv::ConvTap> taps;
  h->sched.commit(&taps, displace);
  h->ctx_ready.assign(h->cfg.layers, false);
  if (!taps.empty()) {
    const int K = h->cfg.conv_kernel;
    const int n_mem = (int)taps.size() / K;
    const size_t esz = h->L.esize, D = h->cfg.head_dim;
    for (int l = 0; l < h->cfg.layers; ++l) {
      bkv::ConvArgs c{};
      for (size_t i = 0; i < taps.size(); ++i) {
        const size_t tok0 = (size_t)taps[i].frame * h->L.Tf;
        c.k_src[i] = h->slot_k(l, taps[i].slot) + tok0 * D * esz;
        c.vt_src[i] = h->slot_vt(l, taps[i].slot) + tok0 * esz;
      }
      c.k_hs = h->slot_k_hs();
      c.vt_hs = h->slot_v_hs();
      c.vt_ld = h->L.Tpad;
      c.k_mem = h->mem_k(l);
      c.k_mem_hs = (long long)h->L.mem_ld * D;
      c.vt_mem = h->mem_vt(l);
      c.vt_mem_hs = (long long)h->L.mem_ld * D;
      c.vt_mem_ld = h->L.mem_ld;
      c.wk = h->conv_w(l, 0);
      c.wv = h->conv_w(l, 1);
      c.H = h->cfg.heads;
      c.D = (int)D;
      c.Tf = h->L.Tf;
      c.tf_pad = h->L.tf_pad;
      c.kernel = K;
      c.n_mem = n_mem;
      hipError_t e = timed(h, K_CONV, stream, [&] { return bkv::launch_conv(c, h->bf16(), stream); });
      if (e != hipSuccess) return device_fail(h, e, "conv launch");
      if (h->vf8()) {                 // the memory's V^T as E4M3 for attention
        bkv::VQuantArgs q{};
        q.vt = h->mem_vt(l);
        q.vt_hs = c.vt_mem_hs;
        q.vt_ld = h->L.mem_ld;
        q.v8 = h->mem_v8(l);
        q.v8_hs = c.vt_mem_hs;
        q.v8_ld = h->L.mem_ld;
        q.vx = h->mem_vx(l);
        q.vx_hs = h->L.mem_ld / bkv::kTokAlign;
        q.H = h->cfg.heads;
        q.n = h->L.mem_ld;            // every memory frame's padded columns (pad stays 0)
        e = timed(h, K_VQUANT, stream, [&] { return bkv::launch_vquant(q, stream); });
        if (e != hipSuccess) return device_fail(h, e, "memory V quantisation launch");
      }
    }
  }
  return BKV_OK;
}

bkv_status bkv_selection(bkv_cache h, int32_t* ids, int32_t cap, int32_t* n, hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (!n) return fail(BKV_ERR_ARG, "null n");
  if (!h->sched.is_open()) return fail(BKV_ERR_STATE, "no open block");
  const int k = h->sched.n_dynamic();
  if (k > 0 && (!ids || cap < k)) return fail(BKV_ERR_ARG, "ids capacity %d < %d", cap, k);
  *n = k;
  if (k == 0) return BKV_OK;
  if ((st = set_device(h)) != BKV_OK) return st;
  hipError_t e = hipMemcpyAsync(ids, h->sel_ids(), sizeof(int) * k, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return device_fail(h, e, "selection copy");
  return BKV_OK;
}

bkv_status bkv_context(bkv_cache h, bkv_segment* segs, int32_t cap, int32_t* n, hipStream_t stream) {
  bkv_status st = check_handle(h, false);
  if (st != BKV_OK) return st;
  if (!n) return fail(BKV_ERR_ARG, "null n");
  const auto& plan = h->sched.segments();
  *n = (int)plan.size();
  if (plan.empty()) return BKV_OK;
  if (!segs || cap < (int)plan.size()) return fail(BKV_ERR_ARG, "segment capacity %d < %zu", cap, plan.size());
  int ids[bkv::kMaxK] = {0};
  const int k = h->sched.n_dynamic();
  if (k > 0) {
    int got = 0;
    if ((st = bkv_selection(h, ids, bkv::kMaxK, &got, stream)) != BKV_OK) return st;
  }
  for (size_t i = 0; i < plan.size(); ++i) {
    const auto& p = plan[i];
    segs[i].kind = p.kind;
    segs[i].tokens = p.tokens;
    if (p.dyn >= 0) {
      segs[i].id = ids[p.dyn];
      if (h->ctx_mode()) {            // the run's first position + frames x rank by stream id
        int rank = 0;
        for (int j = 0; j < k; ++j) rank += ids[j] < ids[p.dyn];
        segs[i].t0 = (int32_t)(p.t0 + (int64_t)rank * h->cfg.frames_per_block);
      } else {
        segs[i].t0 = (int32_t)h->sched.block_t0(ids[p.dyn]);
      }
    } else {
      segs[i].id = (int32_t)p.id;
      segs[i].t0 = (int32_t)p.t0;
      if (h->conv_abs() && p.kind != bkv::SEG_MEMORY) segs[i].t0 = (int32_t)(p.id * h->cfg.frames_per_block);
    }
  }
  return BKV_OK;
}

bkv_status bkv_stats(bkv_cache h, bkv_stats_t* out) {
  if (!h || !out) return fail(BKV_ERR_ARG, "null handle or out");
  out->block = h->sched.block();
  out->open = h->sched.is_open() ? 1 : 0;
  out->n_segments = (int32_t)h->sched.segments().size();
  out->n_keys = h->sched.context_tokens();
  out->last_evicted = h->sched.last_evicted();
  out->bank_count = (int32_t)h->sched.bank_count();
  out->memory_count = h->sched.memory_count();
  out->workspace_bytes = h->L.total;
  out->split_attends = h->split_attends;
  return BKV_OK;
}

bkv_status bkv_export_segment(bkv_cache h, int32_t layer, int32_t seg, void* k_out, void* v_out,
                              hipStream_t stream) {
  bkv_status st = check_handle(h);
  if (st != BKV_OK) return st;
  if (!h->sched.is_open()) return fail(BKV_ERR_STATE, "no open block");
  if (layer < 0 || layer >= h->cfg.layers) return fail(BKV_ERR_ARG, "layer %d out of range", layer);
  const auto& segs = h->sched.segments();
  if (seg < 0 || seg >= (int)segs.size()) return fail(BKV_ERR_ARG, "segment %d out of range", seg);
  if (!k_out || !v_out) return fail(BKV_ERR_ARG, "null output");
  const auto& p = segs[seg];
  if (p.kind == bkv::SEG_CURRENT && !h->sched.attended(layer))
    return fail(BKV_ERR_STATE, "current block of layer %d not written yet", layer);
  if ((st = set_device(h)) != BKV_OK) return st;
  if (h->ctx_mode() && !h->ctx_ready[layer]) {
    if ((st = gather_context(h, layer, stream)) != BKV_OK) return st;
  }
  bkv::ExportArgs a{};
  a.seg = h->seg_arg(layer, p);
  a.sel_slots = h->sel_slots();
  a.slot_base = h->layer_kv(layer);
  a.slot_bytes = (long long)h->L.slot_bytes;
  a.slot_v_off = (long long)h->slot_va_off();
  a.slot_k_hs = h->slot_k_hs();
  a.slot_v_hs = h->slot_v_hs();
  a.slot_v_ld = h->L.Tpad;
  a.kf8 = h->kf8() ? 1 : 0;
  a.slot_kx_off = (long long)h->L.slot_kx_off;
  a.slot_kx_hs = h->slot_kx_hs();
  a.vf8 = h->vf8() ? 1 : 0;
  a.slot_vx_off = (long long)h->L.slot_vx_off;
  a.slot_vx_hs = h->slot_kx_hs();
  a.k_out = k_out;
  a.v_out = v_out;
  a.H = h->cfg.heads;
  a.D = h->cfg.head_dim;
  hipError_t e = timed(h, K_EXPORT, stream, [&] { return bkv::launch_export(a, h->bf16(), stream); });
  if (e != hipSuccess) return device_fail(h, e, "export launch");
  return BKV_OK;
}

bkv_status bkv_probe_mfma(int32_t workgroups, int32_t iters, double* tflops, hipStream_t stream) {
  if (workgroups < 1 || iters < 1 || !tflops) return fail(BKV_ERR_ARG, "workgroups and iters must be >= 1, tflops non-null");
  float* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&sink, sizeof(float));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = bkv::launch_mfma_probe(workgroups, 1, sink, stream);   // warm the code path
  if (e == hipSuccess) e = hipEventRecord(e0, stream);
  if (e == hipSuccess) e = bkv::launch_mfma_probe(workgroups, iters, sink, stream);
  if (e == hipSuccess) e = hipEventRecord(e1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (e != hipSuccess) return fail(BKV_ERR_DEVICE, "MFMA probe: %s", hipGetErrorString(e));
  *tflops = (double)workgroups * 8.0 * iters * 8.0 * 32768.0 / (ms * 1e-3) / 1e12;
  return BKV_OK;
}

bkv_status bkv_profile_start(bkv_cache h, int32_t max_launches) {
  if (!h) return fail(BKV_ERR_ARG, "null handle");
  if (h->prof.on) return fail(BKV_ERR_STATE, "a profile is already recording");
  if (max_launches < 1) return fail(BKV_ERR_ARG, "max_launches must be >= 1");
  bkv_status st = set_device(h);
  if (st != BKV_OK) return st;
  h->prof.ev.assign(2 * (size_t)max_launches, nullptr);
  h->prof.tag.assign(max_launches, -1);
  for (auto& e : h->prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      profile_release(h);
      return fail(BKV_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  h->prof.cap = max_launches;
  h->prof.used = 0;
  h->prof.on = true;
  return BKV_OK;
}

bkv_status bkv_profile_stop(bkv_cache h, bkv_kernel_time* out, int32_t cap, int32_t* n) {
  if (!h || !n) return fail(BKV_ERR_ARG, "null handle or n");
  if (!h->prof.on) return fail(BKV_ERR_STATE, "no profile is recording");
  double tot[K_COUNT] = {0}, mx[K_COUNT] = {0};
  int64_t cnt[K_COUNT] = {0};
  bkv_status st = set_device(h);
  if (st != BKV_OK) {
    profile_release(h);
    return st;
  }
  auto& p = h->prof;
  if (p.used > 0) {
    hipError_t r = hipEventSynchronize(p.ev[2 * p.used - 1]);
    if (r != hipSuccess) {
      profile_release(h);
      return fail(BKV_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorString(r));
    }
  }
  for (int i = 0; i < p.used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) continue;
    tot[p.tag[i]] += ms;
    if (ms > mx[p.tag[i]]) mx[p.tag[i]] = ms;
    cnt[p.tag[i]]++;
  }
  profile_release(h);
  int k = 0;
  for (int t = 0; t < K_COUNT; ++t) k += cnt[t] > 0;
  *n = k;
  if (k > cap || (k > 0 && !out)) return fail(BKV_ERR_ARG, "capacity %d < %d kernels", cap, k);
  int j = 0;
  for (int t = 0; t < K_COUNT; ++t) {
    if (!cnt[t]) continue;
    std::memset(&out[j], 0, sizeof(bkv_kernel_time));
    std::snprintf(out[j].kernel, sizeof(out[j].kernel), "%s", kKernelNames[t]);
    out[j].launches = cnt[t];
    out[j].total_ms = tot[t];
    out[j].max_ms = mx[t];
    ++j;
  }
  return BKV_OK;
}

}  // extern "C"
