// extern "C" boundary of the library.  Every entry point catches everything,
// stores a message and returns a status code (declared in include/chunkattn.h).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>

#include "../../include/chunkattn.h"
#include "kernels.h"
#include "kv_write.h"
#include "manager.h"

using chunkattn::Error;

// The plan of the tree as it will be after the next append of one token to
// every live sequence: built by the call that has just enqueued a step, after
// its launch, so the host builds it while the GPU runs that step.
struct Prebuild {
  // the tree version it was built from and the sequences that append
  uint64_t base_version = 0;
  std::vector<int64_t> ids;
  // the result
  bool ok = false;
  chunkattn::Plan plan;
  int cf_auto = 0, plan_cf_group = 0;
  double ms = 0.0;
  // the workspace the plan's table was copied into, after the step that
  // built it (null: not copied, or overwritten since).  That copy holds each
  // sequence's last chunk at its fill count before the appends, so it
  // becomes the current table once their fill counts are stored (by the
  // step's own blocks, or with the K/V writes).
  void* uploaded_ws = nullptr;
};

static_assert(CA_NOALLOC_SCRATCH_BYTES == chunkattn::kStaticScratchBytes, "the header states the scratch size");

// Byte offsets of a plan's arrays in the workspace: the device table
// (records, chunk refs, row and partial lists, arrival counters), then the
// partial results; table_bytes is what an upload copies, total the size.
struct Layout {
  size_t cf = 0, sf = 0, refs = 0, qrow = 0, seqparts = 0, partlist = 0, arrivals = 0;
  size_t table_bytes = 0, part_o = 0, part_ms = 0, total = 0;
};

struct ca_ctx {
  int heads = 0, head_dim = 0, chunk = 0, flags = 0;
  chunkattn::Manager mgr;
  void* pool = nullptr;
  bool pool_attached = false;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int cf_group = 0, sf_group = 0;  // 0: chosen per plan (auto_cf_group, sf_min_tasks)
  int cf_auto = 8;                 // the last automatic choice
  int plan_cf_group = 8;           // the group the current plan was built with
  int fused_merge = 2;              // CA_OPT_FUSED_MERGE: 0 two launches, 1 one launch, 2 chosen per plan
  int merge_poll_limit = 0;         // CA_OPT_MERGE_POLL_LIMIT (0: the kernels' own bound)
  unsigned decode_epoch = 0;        // ca_decode_step launches that grew chunks in the kernel
  int fail_ops = 0;                 // CA_OPT_FAIL_DEVICE_OPS: device operations left to fail
  int fail_after = 0;               // CA_OPT_FAIL_AFTER_DEVICE_OPS: ones that succeed first
  bool prebuild_on = true;          // CA_OPT_PREBUILD_PLAN
  Prebuild pre;
  int64_t prebuilt_plans = 0;       // structural appends that found their plan built ahead
  bool broken = false;              // a device operation after a tree change failed

  // plan cache: rebuilt after the tree changes, uploaded when stale
  chunkattn::Plan plan;
  bool plan_valid = false;
  bool fills_stale = false;  // plan structure current, chunk fills grew since
  int64_t fill_refreshes = 0, table_uploads = 0, patched_appends = 0;
  // The device copy of the table: the workspace it was uploaded to (the
  // caller's, or a device's static scratch) and the tree version it holds.
  uint64_t version = 1, uploaded_version = 0;
  void* uploaded_ws = nullptr;
  int scratch_dev = -1;             // device whose static scratch uploaded_ws is, or -1
  Layout lay;                       // where the plan's arrays sit in the workspace
  int64_t rebuilds = 0;
  double last_rebuild_ms = 0.0;

  // pinned staging for the table upload, a ring of three buffers: each event
  // marks when the copy out of its buffer has finished, so a buffer is
  // rewritten without waiting on the most recent uploads.  The buffers are
  // three equal parts of the caller's pinned memory (ca_attach_staging) or,
  // when the caller lent none, the library's own: allocated at the first
  // upload, at least kMinStageBytes each and twice the table, so that a tree
  // growing in a decode loop rarely meets a pinned allocation (hipHostFree
  // and hipHostMalloc took 5-6 ms in one such step on MI355X, where the
  // step's kernels take 0.1 ms).
  static constexpr int kStages = 3;
  static constexpr size_t kMinStageBytes = size_t{1} << 20;
  void* stage[kStages] = {nullptr, nullptr, nullptr};
  size_t stage_bytes[kStages] = {0, 0, 0};
  hipEvent_t stage_done[kStages] = {nullptr, nullptr, nullptr};
  bool stage_pending[kStages] = {false, false, false};
  int stage_next = 0;
  void* lent_stage = nullptr;       // the caller's pinned staging, or null
  size_t lent_stage_bytes = 0;

  std::string err;

  ca_ctx(int H, int D, int C, int f) : heads(H), head_dim(D), chunk(C), flags(f),
                                       mgr(C, (f & CA_CREATE_UNSHARED) == 0) {}
  ~ca_ctx() {
    for (int b = 0; b < kStages; ++b) {
      if (stage_done[b]) {
        if (stage_pending[b]) (void)hipEventSynchronize(stage_done[b]);
        (void)hipEventDestroy(stage_done[b]);
      }
      if (stage[b] && lent_stage == nullptr) (void)hipHostFree(stage[b]);
    }
  }
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int fail(ca_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) throw Error(CA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void touch(ca_ctx* c) {
  c->plan_valid = false;
  c->version += 1;
}

// After appends: if they only grew chunks in place, the plan keeps its shape
// and only its fill counts are refreshed; otherwise it is rebuilt.
void touch_after_append(ca_ctx* c) {
  if (c->plan_valid && c->mgr.fills_only()) {
    c->fills_stale = true;
    c->version += 1;
  } else {
    touch(c);
  }
}

// Which context's table each device's static scratch holds (the last one
// uploaded there); a context that finds another owner uploads again.
std::mutex g_scratch_mu;
const ca_ctx* g_scratch_owner[chunkattn::kMaxScratchDevices] = {};

bool scratch_owned_by(const ca_ctx* c) {
  if (c->scratch_dev < 0) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_owner[c->scratch_dev] == c;
}

// The device table in workspace `ws` holds the current tree.
bool table_current_in(const ca_ctx* c, const void* ws) {
  if (ws == nullptr || c->uploaded_version != c->version || c->uploaded_ws != ws) return false;
  return c->scratch_dev < 0 || scratch_owned_by(c);
}

// Some device table (at uploaded_ws) holds the current tree: appends can
// patch fill counts there instead of forcing a new upload.
bool device_table_current(const ca_ctx* c) { return table_current_in(c, c->uploaded_ws); }

// After a failed device operation: the next step uploads the table again
// (which also clears the arrival counters and the fill tags).
void mark_table_stale(ca_ctx* c) { c->uploaded_version = 0; }

// Test knobs (CA_OPT_FAIL_DEVICE_OPS, CA_OPT_FAIL_AFTER_DEVICE_OPS): once
// fail_after more device operations have gone out, the next fail_ops fail as
// a HIP error would, before anything is enqueued.
void device_op(ca_ctx* c, const char* what) {
  if (c->fail_ops > 0) {
    if (c->fail_after > 0) {
      c->fail_after -= 1;
      return;
    }
    c->fail_ops -= 1;
    throw Error(CA_E_HIP, std::string(what) + ": injected failure");
  }
}

// Calls that change the tree update host state that a graph replay would
// not: with a device pool they refuse a capturing stream, before anything
// changes.  A stream the runtime cannot query is not capturing; the error
// is cleared here and the call's own device work reports it.
void refuse_capture(const ca_ctx* c, void* stream, const char* what) {
  if (c->pool == nullptr) return;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &st) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  if (st != hipStreamCaptureStatusNone)
    throw Error(CA_E_STATE, std::string(what) + " changes the tree on the host, which a graph replay would not "
                                                "repeat: call it outside the capture (ca_attend can be captured)");
}

void require_usable(const ca_ctx* c) {
  if (c->broken)
    throw Error(CA_E_STATE, "a device operation failed after the tree had changed; the stored K/V no longer "
                            "match the tree: destroy the context");
}

// Chunk refs per chunk-first task when the caller leaves it open.  A
// chunk-first wave walks its chunks one 32-key half after another, each half
// one dependent round trip to memory (all 16 KiB of its tile loads in flight
// together).  The longest such chain should stay within half of the step's
// own streaming time (unique KV bytes at about 6 TB/s), or the chunk-first
// blocks become the step's tail; within that bound larger groups mean fewer
// blocks and partials.  The per-half cost (2.5 us under full load) is
// calibrated on MI355X: 16 tiles per task (8 halves per wave) are the fastest
// choice at 285-335 MB (1024 and 4096 shared tokens, 32 sequences), while 32
// or 64 make the chains the tail at 4096 shared tokens (65.9 and 89.0 us
// against 59.3 us); from about 80 us of streaming, 32 wins (a 2048-token
// prompt shared by 64 or 96 decoding sequences: 95.2 against 98.4 us and
// 138.6 against 141.9 us; 2048 completion tokens at batch 32: 176.8 against
// 180.4 us).  The group counts chunk refs: a 64-key tile (two halves) at
// C >= 64, one half at C = 32, so 32-token chunks take twice as many refs per
// chain, up to the 64 refs an explicit setting allows.
int auto_cf_group(const chunkattn::Plan& p, int heads, int head_dim, int chunk) {
  const double kernel_us = static_cast<double>(p.unique_tokens) * 4.0 * heads * head_dim / 6.0e6;
  const int halves_per_ref = chunk < chunkattn::kTileKeys ? 1 : 2;
  const int refs_per_tile = 2 / halves_per_ref;
  for (int g : {64, 32, 16, 8}) {
    const int refs = g * refs_per_tile;
    if (refs > 64) continue;
    const int halves = halves_per_ref * ((refs + 3) / 4);
    if (halves * 2.5 <= 0.5 * kernel_us) return refs;
  }
  return 4 * refs_per_tile;
}

// Sequence-first tasks a plan should have when the group is left open: the
// blocks of a step (tasks x heads) should fill the chip's resident block
// slots (three 256-thread blocks on each of 256 CUs) about 2.5 times, or the
// last round leaves CUs idle.  Measured on MI355X: 32 sequences with 512
// private tokens each take 50.4 us with 4 refs per task (2048 blocks) and
// 53.0 us with 8 (1024 blocks); the multi-branch tree, whose suffixes of
// 64..1024 tokens give 4096 blocks even with 16 refs per task, takes 200.6 us
// with 16 against 206.9 us with 4 (one partial per sequence instead of up to
// four).
int64_t sf_min_tasks(int heads) {
  constexpr int64_t kResidentBlocks = 3 * 256;
  return (kResidentBlocks * 5 / 2 + heads - 1) / heads;
}

void layout_plan(ca_ctx* c);
int build_for(const ca_ctx* c, chunkattn::Plan* plan, const chunkattn::NextAppend* next);

// The host plan of the current tree, rebuilt if the tree changed shape.
// with_fills: the host plan's fill counts are needed too (an upload, an
// export, stats); a step whose device table is current does not need them.
void ensure_plan(ca_ctx* c, bool with_fills = true) {
  if (c->plan_valid) {
    if (c->fills_stale && with_fills) {
      auto t0 = std::chrono::steady_clock::now();
      c->mgr.refresh_fills(&c->plan);
      c->fills_stale = false;
      c->fill_refreshes += 1;
      c->last_rebuild_ms =
          std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    }
    return;
  }
  auto t0 = std::chrono::steady_clock::now();
  c->cf_auto = build_for(c, &c->plan, nullptr);
  c->plan_cf_group = c->cf_group ? c->cf_group : c->cf_auto;
  c->mgr.clear_structural();
  c->fills_stale = false;
  layout_plan(c);
  c->plan_valid = true;
  c->rebuilds += 1;
  c->last_rebuild_ms =
      std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// Offsets of a plan's arrays in the workspace (and its total size).
Layout layout_of(const chunkattn::Plan& p, int heads, int head_dim) {
  Layout l;
  size_t off = 0;
  l.cf = off;
  off = align_up(off + p.cf_units.size() * sizeof(chunkattn::CfUnit));
  l.sf = off;
  off = align_up(off + p.sf_tasks.size() * sizeof(chunkattn::SfTask));
  l.refs = off;
  off = align_up(off + p.chunk_refs.size() * sizeof(int32_t));
  l.qrow = off;
  off = align_up(off + p.dfs_qrow.size() * sizeof(int32_t));
  l.seqparts = off;
  off = align_up(off + p.seq_parts.size() * sizeof(int32_t));
  l.partlist = off;
  off = align_up(off + p.part_list.size() * sizeof(int32_t));
  // arrival counters of the fused merge: uploaded as zeros with the table,
  // and every step leaves them at zero again
  l.arrivals = off;
  off = align_up(off + p.dfs_seq.size() * static_cast<size_t>(heads) * sizeof(int32_t));
  l.table_bytes = off;
  l.part_o = off;
  off = align_up(off + static_cast<size_t>(p.n_parts) * heads * head_dim * sizeof(float));
  l.part_ms = off;
  off = align_up(off + static_cast<size_t>(p.n_parts) * heads * 2 * sizeof(float));
  l.total = off;
  return l;
}

void layout_plan(ca_ctx* c) { c->lay = layout_of(c->plan, c->heads, c->head_dim); }

// The plan of a tree: the chunk-first group as given, or chosen for the
// plan (built once with the last choice, again if the plan wants another).
// `next`: the tree after those appends.  Returns the automatic choice.
int build_for(const ca_ctx* c, chunkattn::Plan* plan, const chunkattn::NextAppend* next) {
  const bool two_phase = (c->flags & CA_CREATE_NO_CHUNK_FIRST) == 0;
  const int g = c->cf_group ? c->cf_group : c->cf_auto;
  const int64_t sf_min = sf_min_tasks(c->heads);
  c->mgr.build_plan(g, c->sf_group, two_phase, plan, sf_min, next);
  int cf_auto = c->cf_auto;
  if (c->cf_group == 0 && two_phase && plan->shared_chunks > 0) {
    const int want = auto_cf_group(*plan, c->heads, c->head_dim, c->chunk);
    if (want != g) c->mgr.build_plan(want, c->sf_group, two_phase, plan, sf_min, next);
    cf_auto = want;
  }
  return cf_auto;
}

void copy_table(ca_ctx* c, void* stream, void* ws, const chunkattn::Plan& p, const Layout& l,
                bool before_appends = false);
void note_upload(ca_ctx* c, void* ws, int scratch_dev);

// After a batch of one-token appends over every live sequence (a decode
// step) has been enqueued: if the next such batch will change the plan's
// shape (a sequence's last chunk is full or shared, or a chunk of 128 opens
// its second tile), build the plan of that tree now, while the GPU runs the
// work just enqueued; the next batch then takes it instead of rebuilding.
// upload: the step that reads the current table is enqueued already (a
// decode step), so the new table may go to the workspace now.
void prebuild_next(ca_ctx* c, void* stream, bool upload) {
  Prebuild& p = c->pre;
  if (!c->prebuild_on || c->mgr.live() == 0) return;
  if (p.ok && p.base_version == c->version) return;  // already built for this tree
  if (!c->mgr.next_append_structural()) return;
  const auto t0 = std::chrono::steady_clock::now();
  p.ok = false;
  p.uploaded_ws = nullptr;
  p.base_version = c->version;
  p.ids = c->mgr.sequences();
  chunkattn::NextAppend next;
  if (c->mgr.predict_append_batch(p.ids.data(), static_cast<int32_t>(p.ids.size()), &next) && next.structural) {
    c->mgr.stock_for_append(next);
    p.cf_auto = build_for(c, &p.plan, &next);
    p.plan_cf_group = c->cf_group ? c->cf_group : p.cf_auto;
    p.ok = true;
    // Its table goes to the caller's workspace too, ordered after the work
    // just enqueued, when it fits (else the step that needs it uploads it).
    // The device table then no longer holds the current tree.
    const Layout l = layout_of(p.plan, c->heads, c->head_dim);
    if (upload && c->pool != nullptr && c->ws != nullptr && c->ws_bytes >= l.total && c->fail_ops == 0) {
      try {
        copy_table(c, stream, c->ws, p.plan, l, true);
        p.uploaded_ws = c->ws;
      } catch (const Error&) {
        mark_table_stale(c);
      }
    }
  }
  p.ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// Before the appends of `ids` (one token each): whether the plan built ahead
// is the plan of the tree they will make.
bool prebuild_matches(const ca_ctx* c, const int64_t* ids, int32_t n) {
  const Prebuild& p = c->pre;
  if (!p.ok || p.base_version != c->version || static_cast<size_t>(n) != p.ids.size()) return false;
  for (int32_t j = 0; j < n; ++j)
    if (ids[j] != p.ids[j]) return false;
  return true;
}

// After those appends changed the plan's shape: take the plan built ahead.
// Returns whether its table is in the workspace already (copied ahead, and
// nothing uploaded there since): the device table is then noted as current,
// and the caller must store the appends' fill counts into it (fill_patches)
// or mark it stale.
bool adopt_prebuild(ca_ctx* c) {
  std::swap(c->plan, c->pre.plan);
  c->pre.ok = false;
  c->cf_auto = c->pre.cf_auto;
  c->plan_cf_group = c->pre.plan_cf_group;
  c->mgr.clear_structural();
  c->fills_stale = false;
  layout_plan(c);
  c->plan_valid = true;
  c->rebuilds += 1;
  c->prebuilt_plans += 1;
  c->last_rebuild_ms = c->pre.ms;
  const bool ahead = c->pre.uploaded_ws != nullptr && c->pre.uploaded_ws == c->ws && c->ws_bytes >= c->lay.total;
  if (ahead) note_upload(c, c->ws, -1);
  c->pre.uploaded_ws = nullptr;
  return ahead;
}

template <typename T>
void put(char* base, size_t off, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(base + off, v.data(), v.size() * sizeof(T));
}

// The device table of a plan (table_bytes): records, chunk refs, row and
// partial lists, and zeroed arrival counters.  before_appends: the plan is
// of the tree after one token is appended to every sequence; the chunk ref
// that takes each sequence's token (its task's append field) keeps the fill
// count from before that token.
void table_image(const chunkattn::Plan& p, const Layout& l, char* s, bool before_appends = false) {
  std::memset(s, 0, l.table_bytes);
  put(s, l.cf, p.cf_units);
  put(s, l.sf, p.sf_tasks);
  put(s, l.refs, p.chunk_refs);
  put(s, l.qrow, p.dfs_qrow);
  put(s, l.seqparts, p.seq_parts);
  put(s, l.partlist, p.part_list);
  if (!before_appends) return;
  auto* tasks = reinterpret_cast<chunkattn::SfTask*>(s + l.sf);
  auto* refs = reinterpret_cast<int32_t*>(s + l.refs);
  for (size_t t = 0; t < p.sf_tasks.size(); ++t) {
    const int32_t at = tasks[t].append_at;
    if (at < 0) continue;
    // the fill is at least 1 after the append; the row bit stays
    refs[2 * (tasks[t].chunk_begin + at) + 1] -= 1;
    if (at < chunkattn::kSfInline) tasks[t].n_valid[at] -= 1;
  }
}

// Staging bytes for the current table: three parts, each holding the table.
size_t staging_need(const ca_ctx* c) { return ca_ctx::kStages * align_up(c->lay.table_bytes); }


// Copy a plan's device table into workspace ws on the stream, through the
// next staging buffer of the ring.  Throws before enqueueing anything if the
// stream captures or the lent staging is too small.
void copy_table(ca_ctx* c, void* stream, void* ws, const chunkattn::Plan& p, const Layout& l,
                bool before_appends) {
  // A graph would replay the copy from a staging buffer that later uploads
  // rewrite (and waiting for the ring is no call for a capture): a step is
  // captured only once its table is on the device.
  hipStreamCaptureStatus capturing = hipStreamCaptureStatusNone;
  hip_check(hipStreamIsCapturing(static_cast<hipStream_t>(stream), &capturing), "hipStreamIsCapturing");
  if (capturing != hipStreamCaptureStatusNone)
    throw Error(CA_E_STATE, "the chunk table must be uploaded first, which cannot be captured: run one step "
                            "(or ca_prepare) on the tree as it is before capturing");
  const int b = c->stage_next;
  const size_t need = ca_ctx::kStages * align_up(l.table_bytes);
  if (c->lent_stage != nullptr && c->lent_stage_bytes < need)
    throw Error(CA_E_WORKSPACE, "staging of " + std::to_string(need) + " bytes needed, " +
                                    std::to_string(c->lent_stage_bytes) + " attached");
  if (c->stage_pending[b]) {
    hip_check(hipEventSynchronize(c->stage_done[b]), "hipEventSynchronize");
    c->stage_pending[b] = false;
  }
  if (c->lent_stage == nullptr && c->stage_bytes[b] < l.table_bytes) {
    if (c->stage[b]) hip_check(hipHostFree(c->stage[b]), "hipHostFree");
    c->stage[b] = nullptr;
    c->stage_bytes[b] = 0;
    size_t want = align_up(std::max(l.table_bytes * 2, ca_ctx::kMinStageBytes));
    hip_check(hipHostMalloc(&c->stage[b], want, hipHostMallocDefault), "hipHostMalloc");
    c->stage_bytes[b] = want;
  }
  if (!c->stage_done[b])
    hip_check(hipEventCreateWithFlags(&c->stage_done[b], hipEventDisableTiming), "hipEventCreate");
  char* s = static_cast<char*>(c->stage[b]);
  table_image(p, l, s, before_appends);
  // from here on the device copy may be half written: stale until done
  mark_table_stale(c);
  if (ws == c->pre.uploaded_ws) c->pre.uploaded_ws = nullptr;
  device_op(c, "table upload");
  hip_check(hipMemcpyAsync(ws, s, l.table_bytes, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)),
            "hipMemcpyAsync(table)");
  c->stage_next = (b + 1) % ca_ctx::kStages;
  c->stage_pending[b] = true;
  hip_check(hipEventRecord(c->stage_done[b], static_cast<hipStream_t>(stream)), "hipEventRecord");
  c->table_uploads += 1;
}

// After a table copy into ws holding the current plan: the device table is
// current (untagged fill counts, cleared arrival counters).
void note_upload(ca_ctx* c, void* ws, int scratch_dev) {
  c->decode_epoch = 0;
  c->uploaded_version = c->version;
  c->uploaded_ws = ws;
  c->scratch_dev = scratch_dev;
  if (scratch_dev >= 0) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch_owner[scratch_dev] = c;
  }
}

// scratch_dev: the device whose static scratch ws is, or -1 for the caller's
// workspace.
void upload(ca_ctx* c, void* stream, void* ws, int scratch_dev = -1) {
  if (table_current_in(c, ws)) return;
  ensure_plan(c);
  copy_table(c, stream, ws, c->plan, c->lay);
  note_upload(c, ws, scratch_dev);
}

chunkattn::StepArgs step_args(ca_ctx* c, void* ws, const void* q, void* out) {
  char* w = static_cast<char*>(ws);
  const chunkattn::Plan& p = c->plan;
  chunkattn::StepArgs a{};
  a.pool = c->pool;
  a.q = q;
  a.out = out;
  a.cf_units = reinterpret_cast<const int32_t*>(w + c->lay.cf);
  a.sf_tasks = reinterpret_cast<const int32_t*>(w + c->lay.sf);
  a.chunk_refs = reinterpret_cast<const int32_t*>(w + c->lay.refs);
  a.dfs_qrow = reinterpret_cast<const int32_t*>(w + c->lay.qrow);
  a.seq_parts = reinterpret_cast<const int32_t*>(w + c->lay.seqparts);
  a.part_list = reinterpret_cast<const int32_t*>(w + c->lay.partlist);
  a.part_o = reinterpret_cast<float*>(w + c->lay.part_o);
  a.part_ms = reinterpret_cast<float*>(w + c->lay.part_ms);
  a.arrivals = reinterpret_cast<unsigned*>(w + c->lay.arrivals);
  a.heads = c->heads;
  a.dense_parts = p.dense_parts;
  a.part_stride = p.part_stride;
  a.n_cf_units = static_cast<int>(p.cf_units.size());
  a.n_sf_tasks = static_cast<int>(p.sf_tasks.size());
  a.n_seq = static_cast<int>(p.dfs_seq.size());
  a.scale_log2e = static_cast<float>((1.0 / std::sqrt(static_cast<double>(c->head_dim))) * 1.4426950408889634);
  a.app_k = nullptr;
  a.app_v = nullptr;
  a.app_epoch = 0;
  a.half_tiles = c->chunk < chunkattn::kTileKeys ? 1 : 0;
  a.max_polls = c->merge_poll_limit;
  a.row_chunks = p.row_refs > 0 ? 1 : 0;
  return a;
}

// ws, ws_bytes: the workspace the step runs in (the caller's, or the static
// scratch of the allocation-free step, whose size is fixed).
void check_step(ca_ctx* c, const void* q, void* out, const void* ws, size_t ws_bytes, bool fixed_ws = false) {
  if (!c->pool_attached || c->pool == nullptr) throw Error(CA_E_NO_POOL, "no device pool attached");
  if (c->mgr.live() == 0) throw Error(CA_E_EMPTY, "no live sequence");
  if (q == nullptr || out == nullptr) throw Error(CA_E_INVALID_ARG, "q and out must be device pointers");
  ensure_plan(c, !table_current_in(c, ws));
  if (fixed_ws && ws_bytes < c->lay.total)
    throw Error(CA_E_WORKSPACE, "this step needs a workspace of " + std::to_string(c->lay.total) +
                                    " bytes; the static scratch holds " + std::to_string(ws_bytes));
  if (ws == nullptr || ws_bytes < c->lay.total)
    throw Error(CA_E_WORKSPACE, "workspace of " + std::to_string(c->lay.total) + " bytes needed, " +
                                    std::to_string(ws_bytes) + " attached");
  // int32 indexing limits of the kernels
  if (static_cast<int64_t>(c->plan.cf_units.size()) * c->heads > INT32_MAX ||
      static_cast<int64_t>(c->plan.sf_tasks.size()) * c->heads > INT32_MAX ||
      static_cast<int64_t>(c->plan.dfs_seq.size()) * c->heads > INT32_MAX)
    throw Error(CA_E_UNSUPPORTED, "step too large for one launch");
}

// A kernel launch: the injected failure (if any) comes before anything is
// enqueued; a HIP error is reported with its text.
template <typename F>
void launch(ca_ctx* c, const char* what, F&& go) {
  device_op(c, what);
  const int e = go();
  if (e != 0) throw Error(CA_E_HIP, std::string(what) + ": " + hipGetErrorString(static_cast<hipError_t>(e)));
}

// The device table entries that hold one chunk's fill count: its chunk ref
// and, for one of a task's first refs, the copy inline in the task record
// (offsets in int32 units into the workspace, -1 for none).
struct FillPatch {
  int32_t ref_off, task_off, val;
};

// Appends that only grew private chunks in place, on a context whose table is
// already on the device: the write launch stores the new fill counts into the
// table, so the next step needs no upload.  Returns false, and fills nothing,
// otherwise.  out gets one entry per op.
bool fill_patches(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, std::vector<FillPatch>* out) {
  out->clear();
  if (!c->plan_valid || !c->mgr.fills_only() || !device_table_current(c)) return false;
  const chunkattn::Plan& p = c->plan;
  const int32_t refs = static_cast<int32_t>(c->lay.refs / sizeof(int32_t));
  const int32_t tasks = static_cast<int32_t>(c->lay.sf / sizeof(int32_t));
  constexpr int32_t kTaskInts = sizeof(chunkattn::SfTask) / sizeof(int32_t);
  constexpr int32_t kFillField = offsetof(chunkattn::SfTask, n_valid) / sizeof(int32_t);
  for (const chunkattn::KvOp& o : ops) {
    const int32_t k = o.node >= 0 && static_cast<size_t>(o.node) < p.private_ref.size() ? p.private_ref[o.node] : -1;
    if (k < 0) {
      out->clear();
      return false;
    }
    const int32_t task_off =
        p.ref_pos[k] < chunkattn::kSfInline ? tasks + p.ref_task[k] * kTaskInts + kFillField + p.ref_pos[k] : -1;
    const int32_t row = c->mgr.row(o.node) ? chunkattn::kRowBit : 0;
    out->push_back(FillPatch{refs + 2 * k + 1, task_off, c->mgr.tile_fill(o.dst_key0 + o.n_rows, p.ref_sub[k]) | row});
  }
  return true;
}

// After appends that changed the plan's shape and match the plan built
// ahead: take that plan.  If its table was copied ahead into the workspace,
// the appends' fill counts go into it (patches, one per op) and it is current
// once they are stored; if they cannot be patched there, the table is
// uploaded again before the next step.  Returns whether patches were made.
bool take_prebuild(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, std::vector<FillPatch>* patches) {
  patches->clear();
  if (!adopt_prebuild(c)) return false;
  if (fill_patches(c, ops, patches)) return true;
  mark_table_stale(c);
  return false;
}

bool same_ops(const std::vector<chunkattn::KvOp>& a, const std::vector<chunkattn::KvOp>& b) {
  if (a.size() != b.size()) return false;
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i].dst_slot != b[i].dst_slot || a[i].dst_key0 != b[i].dst_key0 || a[i].n_rows != b[i].n_rows ||
        a[i].src_row0 != b[i].src_row0 || a[i].src_slot != b[i].src_slot || a[i].from_pool != b[i].from_pool ||
        a[i].mode != b[i].mode)
      return false;
  return true;
}

// Whether the step's own blocks can store these appends: one token per op
// from the caller's rows, into a row-major chunk or into a tile part that
// already holds keys (a tile part's first write also clears its other keys,
// which only the write launch does).
bool kernel_can_store(const ca_ctx* c, const std::vector<chunkattn::KvOp>& ops) {
  const int64_t part = std::min<int64_t>(c->chunk, chunkattn::kTileKeys);
  for (const chunkattn::KvOp& o : ops) {
    if (o.n_rows != 1 || o.from_pool || o.mode == chunkattn::kOpConvert) return false;
    if (o.mode == chunkattn::kOpTiles && (static_cast<int64_t>(o.dst_slot) * c->chunk + o.dst_key0) % part == 0)
      return false;
  }
  return true;
}

// The pieces of a copy, one per destination 64-key tile: key k of chunk
// slot s is key (s * C + k) mod 64 of tile (s * C + k) / 64 (chunks of 32
// pair up in a tile, chunks of 128 span two).  A split's tail is read by
// global pool key, so its source may span two tiles within one piece: no two
// pieces of a launch write the same tile, and two chunks sharing a tile
// never share a 16-byte unit.  Keys are written in increasing order, so a
// piece that starts a chunk's part of a tile is that part's first write
// since the slot was allocated: it clears the part's other keys (unwritten V
// columns must be finite, they meet zero probabilities).  A row-major chunk
// needs no clearing (its readers never touch rows past the fill).  A
// conversion to tiles is one piece per tile holding the chunk's keys: the
// chunk's part of the tile and how many of its keys are filled.
void tile_pieces(const chunkattn::KvOp& o, int C, std::vector<chunkattn::KvOpDev>* out) {
  constexpr int32_t T = chunkattn::kTileKeys;
  const int32_t part = std::min<int32_t>(C, T);  // keys of one chunk in one tile
  if (o.mode == chunkattn::kOpConvert) {
    for (int32_t done = 0; done < o.n_rows; done += part) {
      const int64_t dg = static_cast<int64_t>(o.dst_slot) * C + done;
      const int32_t key0 = static_cast<int32_t>(dg % T);
      out->push_back(chunkattn::KvOpDev{static_cast<int32_t>(dg / T), key0, std::min(part, o.n_rows - done), 0, 0,
                                        key0, key0 + part, chunkattn::kKvToTiles});
    }
    return;
  }
  const bool rows = o.mode == chunkattn::kOpRows;
  for (int32_t done = 0; done < o.n_rows;) {
    const int64_t dg = static_cast<int64_t>(o.dst_slot) * C + o.dst_key0 + done;
    const int32_t key0 = static_cast<int32_t>(dg % T);
    const int32_t n = std::min<int32_t>(o.n_rows - done, T - key0);
    const int32_t src0 = o.from_pool ? o.src_slot * C + o.src_row0 + done : o.src_row0 + done;
    const bool first = !rows && dg % part == 0;
    out->push_back(chunkattn::KvOpDev{static_cast<int32_t>(dg / T), key0, n, src0, o.from_pool,
                                      first ? key0 : 0, first ? key0 + part : 0,
                                      rows ? chunkattn::kKvRowWrite : chunkattn::kKvTileWrite});
    done += n;
  }
}

// Launch the copies, at most kOpsPerLaunch tile pieces at a time and never
// one op's pieces (at most two: an op writes one chunk) over two launches; an
// op's patches (if any) ride with its launch.  ops_done (if given) counts the
// ops whose launch has gone out, also when a later launch fails.
void launch_kv_ops(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, const void* k, const void* v, void* stream,
                   const std::vector<FillPatch>& patches, size_t* ops_done = nullptr);

void run_kv_ops(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, const void* k, const void* v, void* stream,
                const std::vector<FillPatch>& patches = {}) {
  // Conversions to tiles first, in launches of their own: the copies of the
  // same mutation may read the converted chunks (a split's tail).
  std::vector<chunkattn::KvOp> converts, rest;
  for (const chunkattn::KvOp& o : ops) (o.mode == chunkattn::kOpConvert ? converts : rest).push_back(o);
  if (converts.empty()) {
    launch_kv_ops(c, ops, k, v, stream, patches);
    return;
  }
  if (!patches.empty()) throw Error(CA_E_INTERNAL, "fill patches with conversions");
  launch_kv_ops(c, converts, k, v, stream, {});
  if (!rest.empty()) launch_kv_ops(c, rest, k, v, stream, {});
}

// The launches of a list of copies (no conversion after another copy of the
// same list: conversions come in lists of their own).
void launch_kv_ops(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, const void* k, const void* v, void* stream,
                   const std::vector<FillPatch>& patches, size_t* ops_done) {
  chunkattn::KvOpBatch batch{};
  chunkattn::TablePatches tp{};
  int n = 0;
  size_t in_batch = 0;  // ops before this index are in a launch or in the batch
  if (ops_done) *ops_done = 0;
  // fill patches go to the device table that holds the current tree
  int32_t* table = static_cast<int32_t*>(c->uploaded_ws);
  auto flush = [&] {
    if (n == 0) return;
    launch(c, "kv_write", [&] { return chunkattn::launch_kv_write(c->pool, c->heads, batch, n, k, v, table, tp, stream); });
    if (ops_done) *ops_done = in_batch;
    n = 0;
    tp.n = 0;
  };
  std::vector<chunkattn::KvOpDev> pieces;
  for (size_t i = 0; i < ops.size(); ++i) {
    pieces.clear();
    tile_pieces(ops[i], c->chunk, &pieces);
    if (n + static_cast<int>(pieces.size()) > chunkattn::kOpsPerLaunch) flush();
    for (const chunkattn::KvOpDev& pc : pieces) batch.ops[n++] = pc;
    if (!patches.empty() && !pieces.empty()) {
      const FillPatch& f = patches[i];
      tp.off[tp.n] = f.ref_off;
      tp.val[tp.n++] = f.val;
      if (f.task_off >= 0) {
        tp.off[tp.n] = f.task_off;
        tp.val[tp.n++] = f.val;
      }
    }
    in_batch = i + 1;
  }
  flush();
}

// The K/V writes of appends that have already changed the tree.  If they
// cannot be enqueued, the tree holds tokens that the pool does not: the
// context refuses further work (CA_E_STATE) from then on.
void store_appended(ca_ctx* c, const std::vector<chunkattn::KvOp>& ops, const void* k, const void* v, void* stream,
                    const std::vector<FillPatch>& patches = {}) {
  try {
    run_kv_ops(c, ops, k, v, stream, patches);
  } catch (const Error&) {
    c->broken = true;
    mark_table_stale(c);
    throw;
  }
}

// Whether a step is one launch (merge blocks close the partials grid) or a
// partials launch and a merge launch.  Measured on MI355X (with the automatic
// task groups), the one-launch step wins once a step merges about 3072
// (sequence, head) pairs (1024 shared + 512 private tokens at 32 heads: 96
// sequences 130.5 vs 131.6 us, 128 sequences 169.9 vs 174.0 us; the
// multi-branch tree 200.9 vs 211.8 us), ties at 2048 (64 sequences: 92.1 vs
// 91.8 us) and loses below (32 sequences: 53.5 vs 50.4 us): its coherent
// partial stores and the merge blocks waiting in the tail cost more than the
// second launch saves until the merge launch itself grows with the pair
// count.
constexpr int64_t kOneLaunchPairs = 3072;

bool one_launch(const ca_ctx* c) {
  if (c->fused_merge != 2) return c->fused_merge == 1;
  return static_cast<int64_t>(c->plan.dfs_seq.size()) * c->heads >= kOneLaunchPairs;
}

// Bookkeeping after appends whose fill counts went to the device with the
// writes: the host plan is refreshed lazily, the device copy is current.
void touch_patched(ca_ctx* c) {
  c->patched_appends += 1;
  c->fills_stale = true;
  c->version += 1;
  c->uploaded_version = c->version;
}

// The step's launches.  After any failure the table is uploaded again before
// the next step (which also clears the arrival counters).
void launch_step(ca_ctx* c, const chunkattn::StepArgs& a, void* stream) {
  try {
    if (one_launch(c)) {
      launch(c, "step", [&] { return chunkattn::launch_partials(a, chunkattn::kPartsBoth, true, stream); });
    } else {
      launch(c, "partials", [&] { return chunkattn::launch_partials(a, chunkattn::kPartsBoth, false, stream); });
      launch(c, "merge", [&] { return chunkattn::launch_merge(a, stream); });
    }
  } catch (const Error&) {
    mark_table_stale(c);
    throw;
  }
}

// The static scratch of the allocation-free step on the current device
// (its address is looked up at the first use on that device and kept).
void* static_scratch_ws(int* dev) {
  void* p = nullptr;
  const int e = chunkattn::static_scratch(&p, dev);
  if (e != 0) throw Error(CA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                        hipGetErrorString(static_cast<hipError_t>(e)));
  return p;
}

// One attend step in workspace ws (after check_step).
void attend_in(ca_ctx* c, const void* q, void* out, void* stream, void* ws, int scratch_dev = -1) {
  upload(c, stream, ws, scratch_dev);
  launch_step(c, step_args(c, ws, q, out), stream);
}

#define CA_GUARD(ctx, ...)                                                    \
  do {                                                                         \
    if ((ctx) == nullptr) return CA_E_INVALID_ARG;                             \
    try {                                                                      \
      (ctx)->err.clear();                                                      \
      __VA_ARGS__                                                              \
    } catch (const Error& e) {                                                 \
      return fail((ctx), e.code, e.what());                                    \
    } catch (const std::bad_alloc&) {                                          \
      return fail((ctx), CA_E_INTERNAL, "host out of memory");                 \
    } catch (const std::exception& e) {                                        \
      return fail((ctx), CA_E_INTERNAL, e.what());                             \
    } catch (...) {                                                            \
      return fail((ctx), CA_E_INTERNAL, "unknown error");                      \
    }                                                                          \
  } while (0)

}  // namespace

extern "C" {

size_t ca_slot_bytes(int heads, int head_dim, int chunk_size) {
  if (heads <= 0 || head_dim <= 0 || chunk_size <= 0) return 0;
  // a 64-key tile (pool_tile_halves at head_dim 128) per 64 tokens
  const size_t tile_heads = chunkattn::pool_tile_halves(heads) / (2 * chunkattn::kTileKeys * chunkattn::kHeadDim);
  return static_cast<size_t>(4) * tile_heads * chunk_size * head_dim;
}

int ca_create_ex(int heads, int head_dim, int chunk_size, int flags, ca_ctx** out) {
  if (out == nullptr) return CA_E_INVALID_ARG;
  *out = nullptr;
  if (heads < 1) return CA_E_INVALID_ARG;
  // Any chunk size up to 64 (or 128) for the tree and tables; a device pool
  // needs 32, 64 or 128 (ca_attach_pool).
  if (head_dim != chunkattn::kHeadDim || chunk_size < 1 || (chunk_size > 64 && chunk_size != 128))
    return CA_E_UNSUPPORTED;
  if (flags & ~(CA_CREATE_UNSHARED | CA_CREATE_NO_CHUNK_FIRST)) return CA_E_UNSUPPORTED;
  try {
    *out = new ca_ctx(heads, head_dim, chunk_size, flags);
  } catch (...) {
    return CA_E_INTERNAL;
  }
  return CA_OK;
}

int ca_create(int heads, int head_dim, int chunk_size, ca_ctx** out) {
  return ca_create_ex(heads, head_dim, chunk_size, 0, out);
}

void ca_destroy(ca_ctx* ctx) {
  if (ctx == nullptr) return;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const ca_ctx*& o : g_scratch_owner)
      if (o == ctx) o = nullptr;
  }
  delete ctx;
}

int ca_attach_pool(ca_ctx* ctx, void* dev, int64_t capacity_slots) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (capacity_slots < 0) throw Error(CA_E_INVALID_ARG, "negative capacity");
    if (dev != nullptr && ctx->chunk != 32 && ctx->chunk != 64 && ctx->chunk != 128)
      throw Error(CA_E_UNSUPPORTED, "a device pool needs chunk size 32, 64 or 128");
    if (dev != nullptr && (reinterpret_cast<uintptr_t>(dev) % kAlign) != 0)
      throw Error(CA_E_INVALID_ARG, "pool must be 256-byte aligned");
    // Chunks of 32 pair up in 64-key tiles and a tile spans every head, so
    // the slots are used in pairs: an odd last slot is left out.
    ctx->mgr.set_capacity(ctx->chunk == 32 ? capacity_slots & ~int64_t{1} : capacity_slots);
    ctx->pool = dev;
    ctx->pool_attached = true;
    touch(ctx);
    return CA_OK;
  });
}

int ca_workspace_bytes(ca_ctx* ctx, size_t* out) {
  CA_GUARD(ctx, {
    if (out == nullptr) throw Error(CA_E_INVALID_ARG, "out is NULL");
    ensure_plan(ctx, false);
    *out = ctx->lay.total;
    return CA_OK;
  });
}

int ca_attach_workspace(ca_ctx* ctx, void* dev, size_t bytes) {
  CA_GUARD(ctx, {
    if (dev != nullptr && (reinterpret_cast<uintptr_t>(dev) % kAlign) != 0)
      throw Error(CA_E_INVALID_ARG, "workspace must be 256-byte aligned");
    // appends must not patch fill counts into a workspace the caller took
    // back, nor take a table copied ahead into it
    if (dev != ctx->ws) {
      if (ctx->uploaded_ws == ctx->ws && ctx->scratch_dev < 0) ctx->uploaded_ws = nullptr;
      ctx->pre.uploaded_ws = nullptr;
    }
    ctx->ws = dev;
    ctx->ws_bytes = dev ? bytes : 0;
    return CA_OK;
  });
}

int ca_staging_bytes(ca_ctx* ctx, size_t* out) {
  CA_GUARD(ctx, {
    if (out == nullptr) throw Error(CA_E_INVALID_ARG, "out is NULL");
    ensure_plan(ctx, false);
    *out = staging_need(ctx);
    return CA_OK;
  });
}

int ca_attach_staging(ca_ctx* ctx, void* host, size_t bytes) {
  CA_GUARD(ctx, {
    if (host != nullptr && (reinterpret_cast<uintptr_t>(host) % kAlign) != 0)
      throw Error(CA_E_INVALID_ARG, "staging must be 256-byte aligned");
    // copies still reading the old buffers finish first: the caller may
    // free them once this returns
    for (int b = 0; b < ca_ctx::kStages; ++b) {
      if (ctx->stage_pending[b]) {
        hip_check(hipEventSynchronize(ctx->stage_done[b]), "hipEventSynchronize");
        ctx->stage_pending[b] = false;
      }
      if (ctx->stage[b] && ctx->lent_stage == nullptr) hip_check(hipHostFree(ctx->stage[b]), "hipHostFree");
      ctx->stage[b] = nullptr;
      ctx->stage_bytes[b] = 0;
    }
    ctx->lent_stage = host;
    ctx->lent_stage_bytes = host ? bytes : 0;
    if (host != nullptr) {
      const size_t part = bytes / ca_ctx::kStages / kAlign * kAlign;
      for (int b = 0; b < ca_ctx::kStages; ++b) {
        ctx->stage[b] = static_cast<char*>(host) + b * part;
        ctx->stage_bytes[b] = part;
        // the events are made here, so that steps never create any
        if (!ctx->stage_done[b])
          hip_check(hipEventCreateWithFlags(&ctx->stage_done[b], hipEventDisableTiming), "hipEventCreate");
      }
    }
    ctx->stage_next = 0;
    return CA_OK;
  });
}

int ca_set_option(ca_ctx* ctx, int option, int value) {
  CA_GUARD(ctx, {
    if (option == CA_OPT_CF_CHUNKS_PER_TASK) {
      if (value < 0 || value > 64) throw Error(CA_E_INVALID_ARG, "chunk-first group must be 0 (auto) or 1..64");
      ctx->cf_group = value;
    } else if (option == CA_OPT_SF_CHUNKS_PER_TASK) {
      if (value < 0 || value > 256) throw Error(CA_E_INVALID_ARG, "sequence-first group must be 0 (auto) or 1..256");
      ctx->sf_group = value;
    } else if (option == CA_OPT_MERGE_POLL_LIMIT) {
      if (value < 0) throw Error(CA_E_INVALID_ARG, "merge poll limit must be >= 0");
      ctx->merge_poll_limit = value;
    } else if (option == CA_OPT_FUSED_MERGE) {
      if (value < 0 || value > 2) throw Error(CA_E_INVALID_ARG, "fused merge is 0, 1 or 2 (automatic)");
      ctx->fused_merge = value;
    } else if (option == CA_OPT_ROW_APPENDS) {
      if (value < 0 || value > 1) throw Error(CA_E_INVALID_ARG, "row appends is 0 or 1");
      ctx->mgr.set_row_appends(value != 0);
      return CA_OK;  // chunks made from now on
    } else if (option == CA_OPT_PREBUILD_PLAN) {
      if (value < 0 || value > 1) throw Error(CA_E_INVALID_ARG, "prebuild is 0 or 1");
      ctx->prebuild_on = value != 0;
      return CA_OK;  // the plan is unaffected
    } else if (option == CA_OPT_FAIL_DEVICE_OPS) {
      if (value < 0) throw Error(CA_E_INVALID_ARG, "failure count must be >= 0");
      ctx->fail_ops = value;
      return CA_OK;  // the plan is unaffected
    } else if (option == CA_OPT_FAIL_AFTER_DEVICE_OPS) {
      if (value < 0) throw Error(CA_E_INVALID_ARG, "operation count must be >= 0");
      ctx->fail_after = value;
      return CA_OK;
    } else {
      throw Error(CA_E_UNSUPPORTED, "unknown option");
    }
    touch(ctx);
    return CA_OK;
  });
}

int ca_insert(ca_ctx* ctx, int64_t seq_id, const int32_t* tokens, int32_t n, const void* k_dev,
              const void* v_dev, void* stream, int32_t* n_matched) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (!ctx->pool_attached) throw Error(CA_E_NO_POOL, "attach a pool (or a NULL pool) first");
    if (n < 1 || tokens == nullptr) throw Error(CA_E_INVALID_ARG, "insert needs n >= 1 host tokens");
    const bool device = ctx->pool != nullptr;
    if (device && (k_dev == nullptr || v_dev == nullptr))
      throw Error(CA_E_INVALID_ARG, "k_dev and v_dev are required when a device pool is attached");
    refuse_capture(ctx, stream, "ca_insert");
    int32_t matched = 0;
    if (!device) {
      matched = ctx->mgr.insert(seq_id, tokens, n, nullptr);
    } else {
      // The copies go out before the tree changes, so a copy that cannot be
      // enqueued leaves the tree as it was.  Conversions of row-major chunks
      // to tiles (chunks this insert shares or splits) come first, in
      // launches of their own; if some went out and a later launch fails,
      // the tree records those chunks' new layout (same tokens, same K/V)
      // and nothing else.
      std::vector<chunkattn::KvOp> ops, converts, rest, done;
      matched = ctx->mgr.insert_ops(seq_id, tokens, n, &ops);
      for (const chunkattn::KvOp& o : ops) (o.mode == chunkattn::kOpConvert ? converts : rest).push_back(o);
      size_t converted = 0;
      try {
        if (!converts.empty()) launch_kv_ops(ctx, converts, k_dev, v_dev, stream, {}, &converted);
        if (!rest.empty()) launch_kv_ops(ctx, rest, k_dev, v_dev, stream, {});
      } catch (const Error&) {
        if (converted > 0) {
          ctx->mgr.mark_tiles(std::vector<chunkattn::KvOp>(converts.begin(), converts.begin() + converted));
          touch(ctx);
        }
        throw;
      }
      ctx->mgr.insert(seq_id, tokens, n, &done);
      if (!same_ops(done, ops)) {
        ctx->broken = true;
        touch(ctx);
        throw Error(CA_E_INTERNAL, "insert: the tree took other slots than its copies wrote");
      }
    }
    touch(ctx);
    if (n_matched) *n_matched = matched;
    return CA_OK;
  });
}

int ca_append(ca_ctx* ctx, int64_t seq_id, const int32_t* tokens, int32_t n, const void* k_dev,
              const void* v_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (!ctx->pool_attached) throw Error(CA_E_NO_POOL, "attach a pool (or a NULL pool) first");
    if (n < 1 || tokens == nullptr) throw Error(CA_E_INVALID_ARG, "append needs n >= 1 host tokens");
    const bool device = ctx->pool != nullptr;
    if (device && (k_dev == nullptr || v_dev == nullptr))
      throw Error(CA_E_INVALID_ARG, "k_dev and v_dev are required when a device pool is attached");
    refuse_capture(ctx, stream, "ca_append");
    std::vector<chunkattn::KvOp> ops;
    std::vector<FillPatch> patches;
    ctx->mgr.append(seq_id, tokens, n, &ops);
    if (device && fill_patches(ctx, ops, &patches))
      touch_patched(ctx);
    else
      touch_after_append(ctx);
    if (device) store_appended(ctx, ops, k_dev, v_dev, stream, patches);
    return CA_OK;
  });
}

int ca_append_batch(ca_ctx* ctx, int32_t n, const int64_t* seq_ids, const int32_t* tokens, const void* k_dev,
                    const void* v_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (!ctx->pool_attached) throw Error(CA_E_NO_POOL, "attach a pool (or a NULL pool) first");
    if (n < 1 || seq_ids == nullptr || tokens == nullptr) throw Error(CA_E_INVALID_ARG, "append batch needs n >= 1");
    const bool device = ctx->pool != nullptr;
    if (device && (k_dev == nullptr || v_dev == nullptr))
      throw Error(CA_E_INVALID_ARG, "k_dev and v_dev are required when a device pool is attached");
    refuse_capture(ctx, stream, "ca_append_batch");
    std::vector<chunkattn::KvOp> ops;
    std::vector<FillPatch> patches;
    const bool prebuilt = prebuild_matches(ctx, seq_ids, n);
    ctx->mgr.append_batch(seq_ids, tokens, n, &ops);
    if (device && fill_patches(ctx, ops, &patches)) {
      touch_patched(ctx);
    } else {
      touch_after_append(ctx);
      // a table copied ahead takes these fill counts with the K/V writes
      if (prebuilt && !ctx->plan_valid && take_prebuild(ctx, ops, &patches)) touch_patched(ctx);
    }
    if (device) store_appended(ctx, ops, k_dev, v_dev, stream, patches);
    // the attention of this step is still to come (ca_attend): build ahead,
    // but leave the table on the device as it is
    prebuild_next(ctx, stream, false);
    return CA_OK;
  });
}

int ca_remove(ca_ctx* ctx, int64_t seq_id) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    ctx->mgr.remove(seq_id);
    touch(ctx);
    return CA_OK;
  });
}

int ca_prepare(ca_ctx* ctx, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (!ctx->pool_attached || ctx->pool == nullptr) throw Error(CA_E_NO_POOL, "no device pool attached");
    if (ctx->mgr.live() == 0) throw Error(CA_E_EMPTY, "no live sequence");
    ensure_plan(ctx, false);
    if (ctx->ws == nullptr || ctx->ws_bytes < ctx->lay.total)
      throw Error(CA_E_WORKSPACE, "workspace too small");
    upload(ctx, stream, ctx->ws);
    return CA_OK;
  });
}

int ca_attend_phase(ca_ctx* ctx, int phase, const void* q_dev, void* out_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (phase < CA_PHASE_CHUNK_FIRST || phase > CA_PHASE_PARTIALS) throw Error(CA_E_INVALID_ARG, "unknown phase");
    check_step(ctx, q_dev, out_dev, ctx->ws, ctx->ws_bytes);
    upload(ctx, stream, ctx->ws);
    chunkattn::StepArgs a = step_args(ctx, ctx->ws, q_dev, out_dev);
    const int part = phase == CA_PHASE_CHUNK_FIRST      ? chunkattn::kPartsChunkFirst
                     : phase == CA_PHASE_SEQUENCE_FIRST ? chunkattn::kPartsSequenceFirst
                                                        : chunkattn::kPartsBoth;
    try {
      if (phase == CA_PHASE_MERGE)
        launch(ctx, "merge", [&] { return chunkattn::launch_merge(a, stream); });
      else
        launch(ctx, "partials", [&] { return chunkattn::launch_partials(a, part, false, stream); });
    } catch (const Error&) {
      mark_table_stale(ctx);
      throw;
    }
    return CA_OK;
  });
}

int ca_attend(ca_ctx* ctx, const void* q_dev, void* out_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    check_step(ctx, q_dev, out_dev, ctx->ws, ctx->ws_bytes);
    attend_in(ctx, q_dev, out_dev, stream, ctx->ws);
    return CA_OK;
  });
}

int ca_attend_noalloc(ca_ctx* ctx, const void* q_dev, void* out_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    int dev = -1;
    void* ws = static_scratch_ws(&dev);
    check_step(ctx, q_dev, out_dev, ws, chunkattn::kStaticScratchBytes, true);
    if (!table_current_in(ctx, ws) && ctx->lent_stage == nullptr)
      throw Error(CA_E_STATE, "the chunk table must be uploaded: attach a staging buffer (ca_attach_staging) first");
    attend_in(ctx, q_dev, out_dev, stream, ws, dev);
    return CA_OK;
  });
}

int ca_decode_step(ca_ctx* ctx, const int32_t* tokens, const void* k_dev, const void* v_dev, const void* q_dev,
                   void* out_dev, void* stream) {
  CA_GUARD(ctx, {
    require_usable(ctx);
    if (!ctx->pool_attached || ctx->pool == nullptr) throw Error(CA_E_NO_POOL, "no device pool attached");
    if (ctx->mgr.live() == 0) throw Error(CA_E_EMPTY, "no live sequence");
    if (tokens == nullptr || k_dev == nullptr || v_dev == nullptr)
      throw Error(CA_E_INVALID_ARG, "tokens, k_dev and v_dev are required");
    if (q_dev == nullptr || out_dev == nullptr) throw Error(CA_E_INVALID_ARG, "q and out must be device pointers");
    refuse_capture(ctx, stream, "ca_decode_step");
    const std::vector<int64_t> ids = ctx->mgr.sequences();
    std::vector<chunkattn::KvOp> ops;
    std::vector<FillPatch> patches;
    const bool prebuilt = prebuild_matches(ctx, ids.data(), static_cast<int32_t>(ids.size()));
    ctx->mgr.append_batch(ids.data(), tokens, static_cast<int32_t>(ids.size()), &ops);
    // The table in the step's workspace holds the tree up to these appends'
    // fill counts: the current table (every token grew its sequence's
    // private last chunk in place), or the one copied ahead for the chunks
    // these appends open.  The fill counts are then stored into it: by the
    // step's own blocks, which also write the tokens, tagging the counts with
    // the epoch (it restarts, with a clean table, before it would wrap), or
    // by the write launch where a token opens a tile part that must be
    // cleared first.
    bool patched = ctx->decode_epoch < chunkattn::kEpochMask && fill_patches(ctx, ops, &patches) &&
                   ctx->uploaded_ws == ctx->ws;
    if (!patched) {
      patches.clear();
      touch_after_append(ctx);
      patched = prebuilt && !ctx->plan_valid && take_prebuild(ctx, ops, &patches);
    }
    const bool in_kernel = patched && kernel_can_store(ctx, ops);
    if (patched) touch_patched(ctx);
    if (in_kernel)
      ctx->decode_epoch += 1;
    else
      store_appended(ctx, ops, k_dev, v_dev, stream, patches);
    try {
      check_step(ctx, q_dev, out_dev, ctx->ws, ctx->ws_bytes);
    } catch (const Error&) {
      // The step cannot run as it is (a larger workspace is needed, or it
      // exceeds the kernels' index range): store the tokens and their fill
      // counts now, as ca_append_batch does, so the tree and the device agree.
      if (in_kernel) store_appended(ctx, ops, k_dev, v_dev, stream, patches);
      throw;
    }
    try {
      upload(ctx, stream, ctx->ws);
      chunkattn::StepArgs a = step_args(ctx, ctx->ws, q_dev, out_dev);
      if (in_kernel) {
        a.app_k = k_dev;
        a.app_v = v_dev;
        a.app_epoch = ctx->decode_epoch;
      }
      launch_step(ctx, a, stream);
    } catch (const Error&) {
      // The tokens were to be written by the step itself: store them with a
      // write launch instead (if that fails too, the context is unusable).
      if (in_kernel) store_appended(ctx, ops, k_dev, v_dev, stream, patches);
      throw;
    }
    prebuild_next(ctx, stream, true);
    return CA_OK;
  });
}

int ca_list_sequences(ca_ctx* ctx, int64_t* ids, int cap) {
  CA_GUARD(ctx, {
    std::vector<int64_t> s = ctx->mgr.sequences();
    if (ids != nullptr)
      for (int i = 0; i < cap && i < static_cast<int>(s.size()); ++i) ids[i] = s[i];
    return static_cast<int>(s.size());
  });
}

int ca_export_table(ca_ctx* ctx, int32_t* rows, int cap_rows, int64_t* dfs_seq_order, int cap_seqs,
                    int* n_rows, int* n_seqs) {
  CA_GUARD(ctx, {
    ensure_plan(ctx);
    const chunkattn::Plan& p = ctx->plan;
    const int nr = static_cast<int>(p.rows.size() / 7), ns = static_cast<int>(p.dfs_seq.size());
    if (n_rows) *n_rows = nr;
    if (n_seqs) *n_seqs = ns;
    if ((rows == nullptr && cap_rows == 0) && (dfs_seq_order == nullptr && cap_seqs == 0)) return CA_OK;
    if (cap_rows < nr || cap_seqs < ns || (nr > 0 && rows == nullptr) || (ns > 0 && dfs_seq_order == nullptr))
      throw Error(CA_E_INVALID_ARG, "output capacity too small");
    if (nr) std::memcpy(rows, p.rows.data(), p.rows.size() * sizeof(int32_t));
    if (ns) std::memcpy(dfs_seq_order, p.dfs_seq.data(), p.dfs_seq.size() * sizeof(int64_t));
    return CA_OK;
  });
}

int ca_export_plan(ca_ctx* ctx, void* buf, size_t cap, size_t* bytes) {
  CA_GUARD(ctx, {
    ensure_plan(ctx);
    if (bytes) *bytes = ctx->lay.table_bytes;
    if (buf == nullptr && cap == 0) return CA_OK;
    if (buf == nullptr || cap < ctx->lay.table_bytes) throw Error(CA_E_INVALID_ARG, "output capacity too small");
    table_image(ctx->plan, ctx->lay, static_cast<char*>(buf));
    return CA_OK;
  });
}

int ca_stats(ca_ctx* ctx, ca_stats_t* out) {
  CA_GUARD(ctx, {
    if (out == nullptr) throw Error(CA_E_INVALID_ARG, "out is NULL");
    ensure_plan(ctx);
    const chunkattn::Plan& p = ctx->plan;
    ca_stats_t s{};
    s.live_sequences = static_cast<int64_t>(ctx->mgr.live());
    s.chunks = ctx->mgr.nodes();
    s.shared_chunks = p.shared_chunks;
    s.unique_tokens = p.unique_tokens;
    s.attended_tokens = p.attended_tokens;
    s.capacity_slots = ctx->mgr.capacity();
    s.free_slots = ctx->mgr.free_slots();
    s.table_rebuilds = ctx->rebuilds;
    s.last_rebuild_ms = ctx->last_rebuild_ms;
    s.cf_tasks = p.cf_tasks;
    s.cf_units = static_cast<int64_t>(p.cf_units.size());
    s.sf_tasks = static_cast<int64_t>(p.sf_tasks.size());
    s.partials = p.n_parts;
    s.cf_chunk_reads = p.cf_chunk_reads;
    s.sf_chunk_reads = p.sf_chunk_reads;
    const int64_t per_tok = 4LL * ctx->heads * ctx->head_dim;
    s.unique_kv_bytes = p.unique_tokens * per_tok;
    s.attended_kv_bytes = p.attended_tokens * per_tok;
    s.shared_tokens = p.shared_tokens;
    s.private_tokens = p.unique_tokens - p.shared_tokens;
    s.fill_refreshes = ctx->fill_refreshes;
    s.table_uploads = ctx->table_uploads;
    s.patched_appends = ctx->patched_appends;
    s.cf_chunks_per_task = ctx->plan_cf_group;
    s.sf_chunks_per_task = ctx->plan.sf_group;
    s.one_launch_step = one_launch(ctx) ? 1 : 0;
    s.prebuilt_plans = ctx->prebuilt_plans;
    s.row_chunks = ctx->mgr.row_chunks();
    *out = s;
    return CA_OK;
  });
}

const char* ca_last_error(ca_ctx* ctx) { return ctx ? ctx->err.c_str() : "NULL context"; }

}  // extern "C"
