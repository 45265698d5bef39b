// Launch interface of the gfx950 kernels (host <-> device argument structs).
//
// Device memory layout used by every kernel (elements of the cache dtype):
//   K rows   [H][ld][D]  -- a head's keys are contiguous rows of D values
//   V^T      [H][D][ld]  -- values stored transposed, so the P.V MFMA reads
//                           8 consecutive keys of one channel as one 16-byte word
// ld (the token stride) is a multiple of 64, so tile loads never leave a row.
// FP8 key cache: K rows hold E4M3 bytes, and an int32 power-of-two exponent
// per (head, 64-token tile) sits at kx [H][ld/64]; V^T stays bf16.
// FP8 KV cache: V^T rows hold E4M3 bytes too, with their own exponents per
// (head, 64-token tile) at vx [H][ld/64].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bkv {

constexpr int kMaxSeg = 20;     // context segments per block (reference+static+dynamic+window+current)
constexpr int kMaxBank = 256;   // PR-Sink bank capacity
constexpr int kMaxK = 8;        // dynamic sinks per block
constexpr int kMaxTaps = 32;    // ConvKV: conv_kernel * memory_frames source frames
constexpr int kTokAlign = 64;   // token-stride alignment of every K / V^T buffer

// bf16 attention work split.  A unit is (head, 256-query tile).  When the
// units leave the last round of kStreamWG workgroups (8 XCDs x 32) part
// idle, the whole rounds run as a plain launch, one unit per workgroup, and
// a second launch of kStreamWG workgroups cuts each remaining unit into up to
// kStreamWG / remaining key-tile parts; the parts' fp32 partial results go
// to split slots (at most kStreamWG), which a third launch merges.
constexpr int kAttnBM = 256;
constexpr int kStreamWG = 256;
constexpr int kStreamPerXcd = kStreamWG / 8;
constexpr size_t kSplitSlotBytes = 8 * 64 * 64 * 4 + 8 * 2 * 64 * 4;   // O registers + (m, l)

// The three tables lie in one allocation (the handle's workspace): kernels
// that pick a table per lane address h and w as element offsets from t.
struct Rope {                   // 3D RoPE tables: (cos, sin) fp32 pairs, built in fp64
  const float2* t;              // [rows][dt/2]; row r <-> temporal position of row r
  const float2* h;              // [grid_h][dh/2]
  const float2* w;              // [grid_w][dw/2]
  int dt, dh, dw;               // channel split, all 0 = no RoPE
  int grid_h, grid_w;
};

// One context segment for attention: keys [0, n).  K rows at k + head*k_hs,
// V^T at v + head*v_hs with row stride v_ld.  dyn >= 0: the segment is a
// retrieved bank block; its slot is sel_slots[dyn] (set on device by the
// retrieval kernel, unknown to the host) and V^T comes from that slot; so
// does K unless k is set (K rotated into the context-K buffer).
struct Seg {
  const void* k;
  const void* v;
  const int* kx;            // FP8 key cache: tile exponents, head h at kx + h*kx_hs
  const int* vx;            // FP8 KV cache: V tile exponents, head h at vx + h*vx_hs
  long long k_hs, v_hs, kx_hs, vx_hs;
  int v_ld, n, dyn, pad_;
};

struct AttnArgs {
  const void* q;            // [T][H][D] caller's queries (rotated and scaled in-kernel)
  void* out;                // [T][H][D]
  int T, H, D;
  int t_row0;               // RoPE t-table row of the current block's frame 0
  float qscale;             // softmax scale * log2(e): the kernels' logits are base 2
  int nseg;
  Rope rope;
  const int* sel_slots;     // device, written by the retrieval kernel
  const char* slot_base;    // layer's slot 0 (bytes); slot s at slot_base + s*slot_bytes
  long long slot_bytes;
  long long slot_v_off;     // byte offset of V^T inside a slot
  long long slot_k_hs, slot_v_hs;
  long long slot_kx_off, slot_kx_hs;   // FP8 key cache: exponents inside a slot
  long long slot_vx_off, slot_vx_hs;   // FP8 KV cache: V exponents inside a slot
  int slot_v_ld;
  int kf8;                  // 1: K is E4M3 with tile exponents (bf16 path only)
  int vf8;                  // 1: V^T is E4M3 with tile exponents too (needs kf8), P V on
                            //    scaled FP8 MFMA with P rounded to E4M3
  int split;                // 1: split slots exist (remainder units may be cut into key parts)
  int unit0;                // first (head, query tile) unit of this launch
  int parts;                // split launch: key parts per remainder unit
  float* part;              // split slots, kSplitSlotBytes each: part p of remainder unit v at p * rU + v
  Seg seg[kMaxSeg];
};

// K/V append with fused RoPE on K (one launch per attend).
struct AppendArgs {
  const void* k_in;         // [T][H][D]
  const void* v_in;         // [T][H][D]
  void* k_rot; long long k_rot_hs; int k_rot_off;   // rotated K rows [H][..][D] at row offset (or null)
  void* k_raw; long long k_raw_hs;                  // raw K rows (ConvKV slot) or null
  void* vt; long long vt_hs; int vt_ld;             // V^T destination
  void* k8; long long k8_hs;                        // FP8 key cache: E4M3 K rows (or null)
  int* kx; long long kx_hs;                         //   and their tile exponents
  void* v8; long long v8_hs; int v8_ld;             // FP8 KV cache: E4M3 V^T (or null; vt, if
  int* vx; long long vx_hs;                         //   also set, gets the bf16 V^T) + exponents
  int T, H, D;
  int t_row0;
  Rope rope;
};

// Fused QKV projection: [q | k | v] = x W^T + b on bf16 MFMA (fp32
// accumulation), with the append kernel's epilogue (K rotated into the
// cache, V into V^T) and q written un-rotated to a scratch buffer.
struct QkvArgs {
  const void* x;            // [T][C] bf16 hidden states
  const void* w;            // [3*H*D][C] bf16: q heads' rows, then k heads', then v heads'
  const void* b;            // [3*H*D] bf16 bias, or null
  int C;                    // hidden width, a multiple of 32
  void* q;                  // [T][H][D] bf16 scratch for the attention kernel
  AppendArgs ap;            // K / V destinations and RoPE, as for the append (k_in, v_in unused)
};

// Retrieval + block-open work, one workgroup.
struct OpenArgs {
  const float* pose_in;     // [P] caller's pose, stored at cur_slot (null: none)
  const float* query;       // [P] pose ranked against the bank (null: pose_in)
  float* pose_store;        // [n_slots][P]
  int P, cur_slot, nbank, k;
  int* sel_ids;             // [k] out
  int* sel_slots;           // [k] out
  float2* ttab;             // t table rows to (re)build, or null
  int t_rows, t_dim;
  long long t_pos0;
  double theta;
  int bank_id[kMaxBank];
  int bank_slot[kMaxBank];
  // Pose-aware bank kept on the device: ids at bank_dev[0..nbank), slots at
  // bank_dev[kMaxBank..], read instead of bank_id / bank_slot when non-null.
  // bank_upd (the same table): upd_pos >= 0 writes (upd_id, upd_slot) there
  // (a block joining a bank with room); with k = 1, the member ranked first
  // is replaced by (upd_id, upd_slot) and its (id, slot) go to victim_out.
  int* bank_dev;
  int upd_pos, upd_id, upd_slot;
  int* victim_out;
};

// ConvKV and context-relative PR-Sink: rotate raw K rows of the context's
// cached segments into the contiguous context-K buffer at context positions.
struct GatherPart {
  const void* src; long long src_hs;   // raw K rows [H][..][D] (dyn >= 0: from the selected slot)
  int dst_off, n, t_row0;              // dst row offset, tokens, t-table row of frame 0
  int dyn;                             // >= 0: retrieved block of rank dyn; t_row0 is then the
                                       // run's first row, plus frames x (its rank by stream id)
  int x_off;                           // FP8 keys: the segment's first tile exponent
};
struct GatherArgs {
  void* dst; long long dst_hs;
  int H, D, nparts, max_n;
  Rope rope;
  const int* sel_ids;                  // retrieved ids and slots (device), n_dyn of each
  const int* sel_slots;
  const char* slot_base; long long slot_bytes, slot_k_hs;
  int n_dyn, frames;
  int kf8;                             // 1: dst holds E4M3 rows, tile exponents at dx
  int* dx; long long dx_hs;            //   exponents [H][dx_hs]
  GatherPart part[kMaxSeg];
};

// ConvKV: depthwise temporal conv (stride = kernel) of raw evicted frames.
struct ConvArgs {
  const void* k_src[kMaxTaps];   // frame i's raw K rows (head 0, first token of the frame)
  const void* vt_src[kMaxTaps];  // frame i's V^T (head 0, row 0, first token column)
  long long k_hs, vt_hs; int vt_ld;
  void* k_mem; long long k_mem_hs;          // memory K rows, frame j at row j*tf_pad
  void* vt_mem; long long vt_mem_hs; int vt_mem_ld;
  const float* wk; const float* wv;         // [H][D][kernel]
  int H, D, Tf, tf_pad, kernel, n_mem;
};

// Inspection copy of one segment to token-major [n][H][D].
struct ExportArgs {
  Seg seg;
  const int* sel_slots;
  const char* slot_base; long long slot_bytes, slot_v_off, slot_k_hs, slot_v_hs; int slot_v_ld;
  long long slot_kx_off, slot_kx_hs; int kf8;   // FP8 key cache: K exported dequantised
  long long slot_vx_off, slot_vx_hs; int vf8;   // FP8 KV cache: V exported dequantised
  void* k_out; void* v_out;
  int H, D;
};

hipError_t launch_rope_table(float2* tab, int rows, int dim, long long pos0, double theta,
                             hipStream_t s);
hipError_t launch_open(const OpenArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, bool bf16, hipStream_t s);
hipError_t launch_qkv(const QkvArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t s);

// Split slots in a file-scope device array instead of the workspace, for
// callers that cannot allocate: kStreamWG slots (the most a split launch
// uses).  static_split_slots() returns the current device's copy (its
// address is looked up once per device); the array keeps the last call's
// contents, and calls that overlap on one device race for it.
constexpr size_t kStaticSplitBytes = kSplitSlotBytes * kStreamWG;
hipError_t static_split_slots(float** slots);

// The bf16 attention shares key tiles across kStreamWG workgroups when its
// (head, kAttnBM-query) units would leave more than 15% of whole-unit rounds
// idle and the workspace holds split slots.
inline bool attention_split(int T, int H, bool slots) {
  const long long units = (long long)((T + kAttnBM - 1) / kAttnBM) * H;
  const long long rounds = (units + kStreamWG - 1) / kStreamWG;
  return slots && units > kStreamWG && rounds * kStreamWG * 100 > units * 115;
}
hipError_t launch_gather(const GatherArgs& a, bool bf16, hipStream_t s);
hipError_t launch_conv(const ConvArgs& a, bool bf16, hipStream_t s);
// FP8 KV cache, ConvKV memory: bf16 V^T [H][D][ld] of n tokens -> E4M3 V^T
// with one exponent per (head, 64-token tile).
struct VQuantArgs {
  const void* vt; long long vt_hs; int vt_ld;
  void* v8; long long v8_hs; int v8_ld;
  int* vx; long long vx_hs;
  int H, n;
};
hipError_t launch_vquant(const VQuantArgs& a, hipStream_t s);
hipError_t launch_export(const ExportArgs& a, bool bf16, hipStream_t s);
hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t s);

}  // namespace bkv
