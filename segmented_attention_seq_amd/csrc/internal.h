// Internal declarations shared by the translation units of libakv.
#pragma once

#include <cstdint>
#include <memory>
#include <string>
#include <utility>
#include <vector>

#include "akv.h"

// std::vector whose resize() leaves new elements uninitialised (the plan builder
// writes every element, in parallel, so the first touch of a large table is spread
// over threads instead of a serial zero fill).
template <class T>
struct DefaultInitAlloc : std::allocator<T> {
  using std::allocator<T>::allocator;
  template <class U> struct rebind { using other = DefaultInitAlloc<U>; };
  template <class U> void construct(U* p) noexcept { ::new (static_cast<void*>(p)) U; }
  template <class U, class... A> void construct(U* p, A&&... a) { ::new (static_cast<void*>(p)) U(std::forward<A>(a)...); }
};
using I32Vec = std::vector<int32_t, DefaultInitAlloc<int32_t>>;

struct akv_plan {
  int32_t bq = 0, bk = 0;
  int64_t T = 0;
  // host tables (layouts documented in akv.h)
  I32Vec tok_pos, tok_drop;
  I32Vec segments;    // 3 per segment
  I32Vec epochs;      // 4 per stretch
  I32Vec versions;    // 3 per version row
  I32Vec ver_run;     // run of each version row (rows of a run move by one shift)
  I32Vec run_delta;   // the shift (row index - append position) of each run
  I32Vec items;       // 2 per item
  I32Vec tile_ptr;    // n_items + 1
  I32Vec tiles;       // k_tile * 4 + class
  I32Vec item_order;
  I32Vec final_tok, final_pos;
  int64_t visible_pairs = 0, p_next = 0, n_full = 0, n_partial = 0, n_runs = 0;
  // device image: contiguous int32 arrays at 256-byte aligned offsets
  std::unique_ptr<uint8_t[]> image;
  uint64_t image_bytes = 0;
  uint64_t off_tok_pos = 0, off_tok_drop = 0, off_ver_src = 0, off_ver_to = 0, off_ver_run = 0,
           off_run_delta = 0, off_item_desc = 0, off_tiles = 0, off_order = 0;
};

namespace akv {

// Per-item descriptor in the device image (8 int32).
enum { ID_QBEGIN = 0, ID_QEND, ID_TB, ID_TE, ID_R, ID_VEROFF, ID_TILE0, ID_TILE1, ID_WORDS };

void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

int build_plan(const akv_op* ops, int64_t n_ops, int32_t bq, int32_t bk, akv_plan** out);

// Kernel launchers (return AKV_OK or AKV_EHIP); arguments are validated by the callers.
struct RopeArgs {
  void* out;
  const void* in;
  void* v_out;          // optional value copy (versions); nullptr if none
  const void* v_in;
  int64_t n_rows;
  int32_t heads, d;
  const int32_t* gather;
  const int32_t* pos_from;
  bool pos_from_by_src;  // pos_from indexed by the gathered source row instead of the output row
  const int32_t* pos_to;
  double base;
  int layout;
  int dtype;
};
int launch_rope(const RopeArgs& a, void* stream);

// Query rotation inside the attention (queries given raw, rotated to their append
// positions on load); off when the queries arrive rotated.
struct RopeQ {
  double rev[64];  // theta_i / (2 pi) for i < d / 2 (d <= 128)
  int on;
  int layout;      // AKV_ROPE_HALF or AKV_ROPE_INTERLEAVED
};

struct AttnArgs {
  const void *q, *k, *v, *k_ver, *v_ver;
  void* out;
  float* lse;
  const int32_t *item_desc, *tiles, *order, *tok_drop, *ver_src, *tok_pos;
  int64_t n_items;
  int32_t hq, hkv, d, bq, bk;
  float scale;
  int dtype;
  RopeQ rq;
  // Version rows rotated at staging time (no version buffers): the plan's run of
  // each version row and shift of each run, and a table of n_runs * d/2 (cos, sin)
  // pairs that the launch fills first (nullptr when the plan has no runs); without
  // `fused` the attention reads k_ver / v_ver.
  bool fused = false;
  const int32_t* ver_run = nullptr;
  const int32_t* run_delta = nullptr;
  int64_t n_runs = 0;
  float* rot_tab = nullptr;
};
int launch_segment_attention(const AttnArgs& a, void* stream);

// Decode split workgroups: one per CU of the MI355X; the batch's gathered keys are
// cut into this many equal ranges.
constexpr int kDecodeWGs = 256;

struct DecodeArgs {
  const void *q, *k, *v;
  const int32_t *indptr, *indices;
  int32_t batch, hq, hkv, d;
  float scale;
  void* out;
  float* lse;
  float* ws;
};
// Workspace floats: one partial (d outputs, max, sum) per query head for each of
// the at most kDecodeWGs + batch - 1 (workgroup, request) overlaps.
uint64_t decode_ws_floats(int32_t batch, int32_t hq, int32_t d);
int launch_decode(const DecodeArgs& a, void* stream);
// The current device's fixed decode scratch (device address and size in floats),
// looked up once per device; for the entry point that allocates nothing.
int decode_static_scratch(float** ptr, uint64_t* floats);

}  // namespace akv
