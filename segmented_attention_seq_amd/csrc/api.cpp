// C ABI of libakv: argument validation, error reporting, dispatch.
#include <cstdint>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <new>
#include <set>
#include <string>

#include "internal.h"

namespace akv {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

}  // namespace akv

using akv::fail;

extern "C" {

const char* akv_status_string(int status) {
  switch (status) {
    case AKV_OK: return "ok";
    case AKV_EINVAL: return "invalid argument";
    case AKV_EOPSEQ: return "invalid op sequence";
    case AKV_EUNSUPPORTED: return "unsupported configuration";
    case AKV_EHIP: return "HIP runtime error";
    case AKV_ENOMEM: return "out of host memory";
    case AKV_ENOSPACE: return "cache index full: remaining slots are locked";
    default: return "unknown status";
  }
}

const char* akv_last_error(void) { return akv::g_last_error.c_str(); }

const char* akv_version(void) { return "akv-mi355x 0.1 (gfx950)"; }

int akv_ops_from_messages(int32_t n_msgs, const int32_t* msg_len, int32_t n_drop,
                          const int32_t* drop_after, const int32_t* drop_target, int32_t n_repos,
                          const int32_t* repos_after, akv_op* ops_out, int64_t ops_cap,
                          int64_t* n_ops_out) {
  if (!n_ops_out) return fail(AKV_EINVAL, "n_ops_out is NULL");
  *n_ops_out = 0;
  if (n_msgs < 0 || n_drop < 0 || n_repos < 0) return fail(AKV_EINVAL, "negative count");
  if ((n_msgs && !msg_len) || (n_drop && (!drop_after || !drop_target)) || (n_repos && !repos_after))
    return fail(AKV_EINVAL, "NULL array with non-zero count");
  try {
    std::vector<int64_t> start(n_msgs + 1, 0);
    for (int32_t k = 0; k < n_msgs; ++k) {
      if (msg_len[k] < 0) return fail(AKV_EINVAL, "message " + std::to_string(k) + " has negative length");
      start[k + 1] = start[k] + msg_len[k];
    }
    std::vector<std::set<int32_t>> targets(n_msgs);
    for (int32_t n = 0; n < n_drop; ++n) {
      const int32_t k = drop_after[n], j = drop_target[n];
      if (k < 0 || k >= n_msgs) return fail(AKV_EOPSEQ, "drop after message " + std::to_string(k) + ": no such message");
      if (j < 0 || j >= n_msgs) return fail(AKV_EOPSEQ, "drop target " + std::to_string(j) + ": no such message");
      if (j > k) return fail(AKV_EOPSEQ, "drop target " + std::to_string(j) + " comes after message " + std::to_string(k));
      targets[k].insert(j);
    }
    std::vector<char> repos(n_msgs, 0);
    for (int32_t n = 0; n < n_repos; ++n) {
      const int32_t k = repos_after[n];
      if (k < 0 || k >= n_msgs) return fail(AKV_EOPSEQ, "reposition after message " + std::to_string(k) + ": no such message");
      repos[k] = 1;
    }
    int64_t need = 0;
    for (int32_t k = 0; k < n_msgs; ++k) {
      need += 1 + repos[k];
      for (int32_t j : targets[k]) need += msg_len[j] > 0;
    }
    *n_ops_out = need;
    if (!ops_out) return AKV_OK;
    if (ops_cap < need) return fail(AKV_EINVAL, "ops_cap too small: need " + std::to_string(need));
    int64_t w = 0;
    for (int32_t k = 0; k < n_msgs; ++k) {
      ops_out[w++] = akv_op{AKV_OP_APPEND, 0, msg_len[k], 0};
      for (int32_t j : targets[k])
        if (msg_len[j] > 0) ops_out[w++] = akv_op{AKV_OP_DROP, 0, start[j], start[j + 1]};
      if (repos[k]) ops_out[w++] = akv_op{AKV_OP_REPOS, 0, 0, 0};
    }
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

int akv_build_visibility(const akv_op* ops, int64_t n_ops, int32_t bq, int32_t bk, akv_plan** out) {
  return akv::build_plan(ops, n_ops, bq, bk, out);
}

int akv_plan_info_get(const akv_plan* p, akv_plan_info* info) {
  if (!p || !info) return fail(AKV_EINVAL, "NULL plan or info");
  info->n_tokens = p->T;
  info->n_segments = (int64_t)p->segments.size() / 3;
  info->n_epochs = (int64_t)p->epochs.size() / 4;
  info->n_versions = (int64_t)p->versions.size() / 3;
  info->n_items = (int64_t)p->items.size() / 2;
  info->n_tiles = (int64_t)p->tiles.size();
  info->n_full = p->n_full;
  info->n_partial = p->n_partial;
  info->visible_pairs = p->visible_pairs;
  info->n_final = (int64_t)p->final_tok.size();
  info->p_next = p->p_next;
  info->bq = p->bq;
  info->bk = p->bk;
  info->device_bytes = p->image_bytes;
  info->n_runs = p->n_runs;
  return AKV_OK;
}

int akv_plan_tables_get(const akv_plan* p, akv_plan_tables* v) {
  if (!p || !v) return fail(AKV_EINVAL, "NULL plan or views");
  v->tok_pos = p->tok_pos.data();
  v->tok_drop = p->tok_drop.data();
  v->segments = p->segments.data();
  v->epochs = p->epochs.data();
  v->versions = p->versions.data();
  v->items = p->items.data();
  v->tile_ptr = p->tile_ptr.data();
  v->tiles = p->tiles.data();
  v->item_order = p->item_order.data();
  v->final_tok = p->final_tok.data();
  v->final_pos = p->final_pos.data();
  v->ver_run = p->ver_run.data();
  v->run_delta = p->run_delta.data();
  return AKV_OK;
}

int akv_plan_upload(const akv_plan* p, void* dev, uint64_t dev_bytes, akv_stream_t stream) {
  if (!p || !dev) return fail(AKV_EINVAL, "NULL plan or device buffer");
  if (dev_bytes < p->image_bytes) return fail(AKV_EINVAL, "device buffer smaller than the plan image");
  hipError_t e = hipMemcpyAsync(dev, p->image.get(), p->image_bytes, hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return fail(AKV_EHIP, std::string("plan upload: ") + hipGetErrorString(e));
  return AKV_OK;
}

void akv_plan_destroy(akv_plan* p) { delete p; }

static int check_rope(int dtype, int32_t heads, int32_t d, int layout, double base) {
  if (dtype != AKV_F32 && dtype != AKV_BF16) return fail(AKV_EINVAL, "dtype must be AKV_F32 or AKV_BF16");
  if (heads < 1) return fail(AKV_EINVAL, "heads must be >= 1");
  if (d < 16 || d > 256 || d % 16) return fail(AKV_EUNSUPPORTED, "RoPE needs d % 16 == 0 and 16 <= d <= 256");
  if (layout != AKV_ROPE_HALF && layout != AKV_ROPE_INTERLEAVED) return fail(AKV_EINVAL, "unknown RoPE layout");
  if (!(base > 1.0) || !std::isfinite(base)) return fail(AKV_EINVAL, "RoPE base must be finite and > 1");
  return AKV_OK;
}

int akv_rope_repos(void* out, const void* in, int dtype, int64_t n_rows, int32_t heads, int32_t d,
                   const int32_t* gather, const int32_t* pos_from, const int32_t* pos_to,
                   double rope_base, int rope_layout, akv_stream_t stream) {
  int st = check_rope(dtype, heads, d, rope_layout, rope_base);
  if (st) return st;
  if (n_rows < 0) return fail(AKV_EINVAL, "n_rows < 0");
  if (n_rows == 0) return AKV_OK;
  if (!out || !in || !pos_to) return fail(AKV_EINVAL, "NULL out, in or pos_to");
  if (gather && out == in) return fail(AKV_EINVAL, "in-place rotation cannot gather");
  akv::RopeArgs a{out, in, nullptr, nullptr, n_rows, heads, d, gather, pos_from, false, pos_to,
                  rope_base, rope_layout, dtype};
  return akv::launch_rope(a, stream);
}

int akv_kv_reuse(void* k_out, void* v_out, const void* k_pool, const void* v_pool, int dtype, int64_t n_rows,
                 int32_t heads, int32_t d, const int32_t* gather, const int32_t* pos_from,
                 const int32_t* pos_to, double rope_base, int rope_layout, akv_stream_t stream) {
  int st = check_rope(dtype, heads, d, rope_layout, rope_base);
  if (st) return st;
  if (n_rows < 0) return fail(AKV_EINVAL, "n_rows < 0");
  if (n_rows == 0) return AKV_OK;
  if (!k_out || !v_out || !k_pool || !v_pool || !gather || !pos_from || !pos_to)
    return fail(AKV_EINVAL, "NULL pointer argument");
  if (k_out == k_pool || v_out == v_pool || k_out == v_out) return fail(AKV_EINVAL, "outputs must not alias the pools");
  akv::RopeArgs a{k_out, k_pool, v_out, v_pool, n_rows, heads, d, gather, pos_from, false, pos_to,
                  rope_base, rope_layout, dtype};
  return akv::launch_rope(a, stream);
}

int akv_rope_apply(const akv_plan* p, const void* dev_plan, void* out, const void* in, int dtype,
                   int32_t heads, int32_t d, double rope_base, int rope_layout, akv_stream_t stream) {
  if (!p || !dev_plan) return fail(AKV_EINVAL, "NULL plan or device plan");
  int st = check_rope(dtype, heads, d, rope_layout, rope_base);
  if (st) return st;
  if (p->T == 0) return AKV_OK;
  if (!out || !in) return fail(AKV_EINVAL, "NULL out or in");
  const auto* base = (const uint8_t*)dev_plan;
  akv::RopeArgs a{out, in, nullptr, nullptr, p->T, heads, d, nullptr, nullptr, false,
                  (const int32_t*)(base + p->off_tok_pos), rope_base, rope_layout, dtype};
  return akv::launch_rope(a, stream);
}

int akv_build_kv_versions(const akv_plan* p, const void* dev_plan, const void* k, const void* v,
                          void* k_ver, void* v_ver, int dtype, int32_t hkv, int32_t d,
                          double rope_base, int rope_layout, akv_stream_t stream) {
  if (!p || !dev_plan) return fail(AKV_EINVAL, "NULL plan or device plan");
  int st = check_rope(dtype, hkv, d, rope_layout, rope_base);
  if (st) return st;
  const int64_t nv = (int64_t)p->versions.size() / 3;
  if (nv == 0) return AKV_OK;
  if (!k || !v || !k_ver || !v_ver) return fail(AKV_EINVAL, "NULL k, v, k_ver or v_ver");
  const auto* base = (const uint8_t*)dev_plan;
  akv::RopeArgs a{k_ver, k, v_ver, v, nv, hkv, d, (const int32_t*)(base + p->off_ver_src),
                  (const int32_t*)(base + p->off_tok_pos), true, (const int32_t*)(base + p->off_ver_to),
                  rope_base, rope_layout, dtype};
  return akv::launch_rope(a, stream);
}

int32_t akv_attention_bq(int32_t hq, int32_t hkv) {
  if (hq < 1 || hkv < 1 || hq % hkv) return 64;
  const int32_t grp = hq / hkv;
  return (grp == 1 || grp == 2 || grp == 4) ? 512 / grp : 64;
}

namespace {

int segment_attention(const akv_plan* p, const void* dev_plan, const void* q, const void* k, const void* v,
                      const void* k_ver, const void* v_ver, void* out, float* lse, int dtype, int32_t hq,
                      int32_t hkv, int32_t d, float scale, const akv::RopeQ& rq, akv_stream_t stream,
                      bool fused = false, float* rot_tab = nullptr) {
  if (!p || !dev_plan) return fail(AKV_EINVAL, "NULL plan or device plan");
  if (dtype != AKV_F32 && dtype != AKV_BF16) return fail(AKV_EINVAL, "dtype must be AKV_F32 or AKV_BF16");
  if (hq < 1 || hkv < 1 || hq % hkv) return fail(AKV_EINVAL, "hq must be a positive multiple of hkv");
  const int32_t grp = hq / hkv;
  if (dtype == AKV_BF16) {
    if (d != 64) return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs d == 64");
    if (p->bk != 64 || (p->bq != 64 && (grp >= 8 || p->bq * grp != 512)))
      return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs a plan with bk == 64 and bq == 64 or 64 * 8 / (hq / hkv)");
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
      return fail(AKV_EUNSUPPORTED, "bf16 segment attention needs hq/hkv in {1, 2, 4, 8}");
  } else {
    if (d < 1 || d > 128) return fail(AKV_EUNSUPPORTED, "f32 segment attention needs d <= 128");
    if (p->bq > 256) return fail(AKV_EUNSUPPORTED, "f32 segment attention needs bq <= 256");
  }
  if (p->T == 0) return AKV_OK;
  if (!q || !k || !v || !out) return fail(AKV_EINVAL, "NULL q, k, v or out");
  if (!fused && !p->versions.empty() && (!k_ver || !v_ver))
    return fail(AKV_EINVAL, "plan has version rows: k_ver/v_ver required");
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)d);
  const auto* base = (const uint8_t*)dev_plan;
  akv::AttnArgs a{q, k, v, k_ver, v_ver, out, lse,
                  (const int32_t*)(base + p->off_item_desc), (const int32_t*)(base + p->off_tiles),
                  (const int32_t*)(base + p->off_order), (const int32_t*)(base + p->off_tok_drop),
                  (const int32_t*)(base + p->off_ver_src), (const int32_t*)(base + p->off_tok_pos),
                  (int64_t)p->items.size() / 2, hq, hkv, d, p->bq, p->bk, scale, dtype, rq};
  if (fused) {
    a.fused = true;
    a.ver_run = (const int32_t*)(base + p->off_ver_run);
    a.run_delta = (const int32_t*)(base + p->off_run_delta);
    a.n_runs = p->n_runs;
    a.rot_tab = rot_tab;
  }
  return akv::launch_segment_attention(a, stream);
}

}  // namespace

int akv_segment_attention(const akv_plan* p, const void* dev_plan, const void* q, const void* k,
                          const void* v, const void* k_ver, const void* v_ver, void* out, float* lse,
                          int dtype, int32_t hq, int32_t hkv, int32_t d, float scale,
                          akv_stream_t stream) {
  akv::RopeQ rq{};
  rq.on = 0;
  return segment_attention(p, dev_plan, q, k, v, k_ver, v_ver, out, lse, dtype, hq, hkv, d, scale, rq, stream);
}

int akv_segment_attention_rope(const akv_plan* p, const void* dev_plan, const void* q_raw, const void* k,
                               const void* v, const void* k_ver, const void* v_ver, void* out, float* lse,
                               int dtype, int32_t hq, int32_t hkv, int32_t d, float scale, double rope_base,
                               int rope_layout, akv_stream_t stream) {
  if (!(rope_base > 1.0) || !std::isfinite(rope_base)) return fail(AKV_EINVAL, "RoPE base must be finite and > 1");
  if (rope_layout != AKV_ROPE_HALF && rope_layout != AKV_ROPE_INTERLEAVED)
    return fail(AKV_EINVAL, "rope_layout must be AKV_ROPE_HALF or AKV_ROPE_INTERLEAVED");
  if (d < 2 || d > 128 || d % 2) return fail(AKV_EUNSUPPORTED, "query rotation needs an even d <= 128");
  akv::RopeQ rq{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d / 2; ++i) rq.rev[i] = std::pow(rope_base, -2.0 * i / d) / two_pi;
  rq.on = 1;
  rq.layout = rope_layout;
  return segment_attention(p, dev_plan, q_raw, k, v, k_ver, v_ver, out, lse, dtype, hq, hkv, d, scale, rq, stream);
}

uint64_t akv_rot_table_bytes(const akv_plan* p, int32_t d) {
  if (!p || d < 2 || d > 128 || d % 2) return 0;
  return (uint64_t)p->n_runs * (uint64_t)(d / 2) * 8;
}

int akv_segment_attention_fused(const akv_plan* p, const void* dev_plan, const void* q_raw, const void* k,
                                const void* v, void* out, float* lse, int dtype, int32_t hq, int32_t hkv,
                                int32_t d, float scale, double rope_base, int rope_layout, void* ws,
                                uint64_t ws_bytes, akv_stream_t stream) {
  if (!p || !dev_plan) return fail(AKV_EINVAL, "NULL plan or device plan");
  if (!(rope_base > 1.0) || !std::isfinite(rope_base)) return fail(AKV_EINVAL, "RoPE base must be finite and > 1");
  if (rope_layout != AKV_ROPE_HALF && rope_layout != AKV_ROPE_INTERLEAVED)
    return fail(AKV_EINVAL, "rope_layout must be AKV_ROPE_HALF or AKV_ROPE_INTERLEAVED");
  // 8 query heads per kv head with 64-token query tiles, or 4, 2, 1 with query tiles
  // of 64 * 8 / (hq / hkv) tokens: the ping-pong kernel
  const bool heads_ok = hkv >= 1 && hq % hkv == 0 &&
                        ((hq == 8 * hkv && p->bq == 64) || ((hq / hkv == 4 || hq / hkv == 2 || hq == hkv) &&
                                                            p->bq * (hq / hkv) == 512));
  if (dtype != AKV_BF16 || d != 64 || !heads_ok)
    return fail(AKV_EUNSUPPORTED, "fused version rotation needs bf16, d == 64, and hq == 8 * hkv with bq == 64 "
                                  "or hq / hkv in {1, 2, 4} with bq == 64 * 8 / (hq / hkv)");
  // the kernel's gathered copies address k and v by 32-bit byte offsets
  if ((uint64_t)p->T * (uint64_t)hkv * (uint64_t)d * 2 > 0xffffffffull)
    return fail(AKV_EUNSUPPORTED, "fused version rotation needs k and v under 4 GiB each");
  const uint64_t need = akv_rot_table_bytes(p, d);
  if (ws_bytes < need || (need && !ws)) return fail(AKV_EINVAL, "rotation table workspace too small");
  akv::RopeQ rq{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d / 2; ++i) rq.rev[i] = std::pow(rope_base, -2.0 * i / d) / two_pi;
  rq.on = 1;
  rq.layout = rope_layout;
  return segment_attention(p, dev_plan, q_raw, k, v, nullptr, nullptr, out, lse, dtype, hq, hkv, d, scale, rq,
                           stream, true, (float*)ws);
}

uint64_t akv_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int64_t max_n) {
  (void)hkv;
  if (batch < 1 || hq < 1 || d < 1 || max_n < 1 || max_n > INT32_MAX) return 0;
  return 4 * akv::decode_ws_floats(batch, hq, d);
}

// Argument checks shared by the two decode entry points (the workspace aside).
static int decode_check(const void* q, const void* k_pool, const void* v_pool, const int32_t* indptr,
                        const int32_t* indices, int32_t batch, int32_t hq, int32_t hkv, int32_t d, int64_t max_n,
                        int dtype, const void* out) {
  if (dtype != AKV_BF16) return fail(AKV_EUNSUPPORTED, "decode attention is bf16 only");
  if (d != 64) return fail(AKV_EUNSUPPORTED, "decode attention needs d == 64");
  if (hq < 1 || hkv < 1 || hq % hkv || hq / hkv > 16)
    return fail(AKV_EUNSUPPORTED, "decode needs hq a multiple of hkv with hq/hkv <= 16");
  if (batch < 0) return fail(AKV_EINVAL, "batch < 0");
  if (batch == 0) return AKV_OK;
  if (!q || !k_pool || !v_pool || !indptr || !indices || !out) return fail(AKV_EINVAL, "NULL pointer argument");
  if (max_n < 1 || max_n > INT32_MAX) return fail(AKV_EINVAL, "max_n must be in [1, 2^31)");
  return AKV_OK;
}

int akv_decode_attention(const void* q, const void* k_pool, const void* v_pool, const int32_t* indptr,
                         const int32_t* indices, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                         int64_t max_n, float scale, int dtype, void* out, float* lse, void* ws,
                         uint64_t ws_bytes, akv_stream_t stream) {
  int st = decode_check(q, k_pool, v_pool, indptr, indices, batch, hq, hkv, d, max_n, dtype, out);
  if (st != AKV_OK || batch == 0) return st;
  if (!ws) return fail(AKV_EINVAL, "NULL pointer argument");
  if (ws_bytes < 4 * akv::decode_ws_floats(batch, hq, d)) return fail(AKV_EINVAL, "decode workspace too small");
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)d);
  akv::DecodeArgs a{q, k_pool, v_pool, indptr, indices, batch, hq, hkv, d, scale, out, lse, (float*)ws};
  return akv::launch_decode(a, stream);
}

int akv_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* indptr,
                                 const int32_t* indices, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                 int64_t max_n, float scale, int dtype, void* out, float* lse,
                                 akv_stream_t stream) {
  int st = decode_check(q, k_pool, v_pool, indptr, indices, batch, hq, hkv, d, max_n, dtype, out);
  if (st != AKV_OK || batch == 0) return st;
  float* ws = nullptr;
  uint64_t cap = 0;
  st = akv::decode_static_scratch(&ws, &cap);
  if (st != AKV_OK) return st;
  const uint64_t need = akv::decode_ws_floats(batch, hq, d);
  if (need > cap)
    return fail(AKV_EINVAL, "decode needs " + std::to_string(4 * need) + " bytes of scratch; the fixed scratch holds " +
                                std::to_string(4 * cap));
  if (!(scale > 0.0f)) scale = 1.0f / std::sqrt((float)d);
  akv::DecodeArgs a{q, k_pool, v_pool, indptr, indices, batch, hq, hkv, d, scale, out, lse, ws};
  return akv::launch_decode(a, stream);
}

}  // extern "C"
