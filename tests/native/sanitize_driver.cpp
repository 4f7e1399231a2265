// Host-only driver for the sanitizer build of libsgg_lora's host code: the
// planner (plan.cpp), the shrink tile choice (tiling.cpp) and the C-ABI entry
// points with their validation (lora_api.hip), linked with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host side.  The kernel launchers are
// replaced by stubs that record the launch and enqueue nothing, and the pinned
// memory lookup by one that maps every buffer to itself, so every entry point
// runs its host path in full on a machine without a GPU.
//
// Protocol: one command per input line, one result line per command.
//   P decode max_chunk override max_loras seg_cap has_lens n lens[n] slots[n]
//       -> rc n_seg chunk n_tok | perm[n_tok] | seg_indptr[cap+1] | seg_slots[cap] | req[n+1]
//   H max_chunk override max_loras seg_cap n lens[n] slots[n]
//       -> rc n_seg chunk n_tok | perm[n_tok] | seg_indptr[cap+1] | seg_slots[cap]
//   U lm_head decode max_chunk override max_loras tok_cap seg_cap req_cap has_lens n
//     lens[n] slots[n] ranks[max_loras] scaling_bits[max_loras]
//       -> rc info[6] | staging[total words]
//   E decode max_chunk L tok_cap seg_cap req_cap has_lens n lens[n] slots[n]
//     ranks[L] scaling_bits[L] R
//       -> rc info[6] | staging[total words] | fused s R n_copy
//          | slot[s] | rank[64]          (the last two only when fused is 1)
//   V   -> "name rc" for each built-in validation case, then "end"
// Every host buffer the library writes is allocated at exactly the size the
// call is told, so an overrun is a heap-buffer-overflow report.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/sgg_lora.h"
#include "../../segmented_gather_gemm_amd/csrc/sgg_kernels.h"

namespace sgg {
// Launch stubs: count the launches, enqueue nothing.
static int g_launches = 0;
hipError_t launch_shrink(const ShrinkParams&, const ShrinkTiling&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_shrink_gemm(const ShrinkParams&, int, int, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_expand(const ExpandParams&, const ExpandTiling&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_embedding(const EmbeddingParams&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_plan_device(const int32_t*, const int32_t*, int32_t, const int32_t*,
                              const float*, int32_t, int32_t, int32_t, int32_t, int64_t, int32_t,
                              const int64_t*, int32_t*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_plan_copy(const int32_t*, int32_t*, int64_t, int32_t*, int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
// The one-launch upload + embedding: its arguments are kept for the E command.
static int g_fused_embeds = 0;
static EmbedUploadParams g_last_embed;
hipError_t launch_plan_copy_embedding(const EmbedUploadParams& p, hipStream_t) {
  ++g_launches;
  ++g_fused_embeds;
  g_last_embed = p;
  return hipSuccess;
}
hipError_t launch_moe_plan(const MoeRouteParams&, int32_t, int32_t, const int64_t*, int32_t*,
                           int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_moe_route(const MoeRouteParams&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int64_t fused_resident_blocks(int, int, int) { return int64_t{1} << 30; }
hipError_t launch_fused(const ShrinkParams&, const ShrinkTiling&, const ExpandParams&,
                        const ExpandTiling&, const FusedSync&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace sgg

// Pinned-memory lookup stub: every host buffer "has" a device mapping at its
// own address, so lora_plan_upload takes its copy-kernel path (stubbed above)
// and completes on the host.
extern "C" hipError_t hipHostGetDevicePointer(void** devPtr, void* hstPtr, unsigned int) {
  *devPtr = hstPtr;
  return hipSuccess;
}

namespace {

std::vector<int32_t> read_ints(std::istringstream& in, int64_t n) {
  std::vector<int32_t> v(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) in >> v[static_cast<size_t>(i)];
  return v;
}

// Exactly-sized heap copy (nullptr for n == 0) so reads past the end trip ASan.
template <typename T>
T* exact(const std::vector<T>& v) {
  if (v.empty()) return nullptr;
  T* p = static_cast<T*>(std::malloc(v.size() * sizeof(T)));
  std::memcpy(p, v.data(), v.size() * sizeof(T));
  return p;
}

void put(std::ostringstream& out, const int32_t* p, int64_t n) {
  out << " |";
  for (int64_t i = 0; i < n; ++i) out << ' ' << p[i];
}

void cmd_plan(std::istringstream& in, bool lm_head) {
  int decode = 0, max_chunk, override, L, cap, has_lens = 1, n;
  if (!lm_head) in >> decode;
  in >> max_chunk >> override >> L >> cap;
  if (!lm_head) in >> has_lens;
  in >> n;
  std::vector<int32_t> lens = has_lens ? read_ints(in, n) : std::vector<int32_t>();
  std::vector<int32_t> slots = read_ints(in, n);
  int64_t s = 0;
  if (has_lens)
    for (int32_t v : lens) s += v > 0 ? v : 0;
  else
    s = n;
  int32_t* pl = exact(lens);
  int32_t* ps = exact(slots);
  int32_t* perm = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (s > 0 ? s : 1)));
  int32_t* ind = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (cap + 1)));
  int32_t* sl = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (cap > 0 ? cap : 1)));
  int32_t* req = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (n + 1)));
  int32_t n_seg = -1, chunk = -1;
  int64_t n_tok = -1;
  int rc;
  if (lm_head)
    rc = lora_plan_lm_head(pl, ps, n, L, max_chunk, override, perm, s, ind, sl, cap, &n_seg,
                           &chunk, &n_tok);
  else
    rc = lora_plan_segments(pl, ps, n, L, decode, max_chunk, override, perm, s, ind, sl, cap,
                            req, &n_seg, &chunk, &n_tok);
  std::ostringstream out;
  out << rc << ' ' << n_seg << ' ' << chunk << ' ' << n_tok;
  if (rc == 0) {
    put(out, perm, n_tok);
    put(out, ind, cap + 1);
    put(out, sl, cap);
    if (!lm_head) put(out, req, n + 1);
  }
  std::cout << out.str() << '\n';
  std::free(pl);
  std::free(ps);
  std::free(perm);
  std::free(ind);
  std::free(sl);
  std::free(req);
}

void cmd_upload(std::istringstream& in) {
  int lm_head, decode, max_chunk, override, L, seg_cap, req_cap, has_lens, n;
  int64_t tok_cap;
  in >> lm_head >> decode >> max_chunk >> override >> L >> tok_cap >> seg_cap >> req_cap >>
      has_lens >> n;
  std::vector<int32_t> lens = has_lens ? read_ints(in, n) : std::vector<int32_t>();
  std::vector<int32_t> slots = read_ints(in, n);
  std::vector<int32_t> ranks = read_ints(in, L);
  std::vector<int32_t> sbits = read_ints(in, L);
  std::vector<float> scal(static_cast<size_t>(L));
  std::memcpy(scal.data(), sbits.data(), sizeof(float) * L);
  const int64_t total = lora_plan_layout(tok_cap, seg_cap, req_cap, L, nullptr);
  int32_t* staging = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * total));
  std::memset(staging, 0xff, sizeof(int32_t) * total);
  int32_t* device = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * total));
  int32_t* pl = exact(lens);
  int32_t* ps = exact(slots);
  int32_t* pr = exact(ranks);
  float* pf = exact(scal);
  int32_t info[6] = {-1, -1, -1, -1, -1, -1};
  int rc;
  if (lm_head)
    rc = lora_plan_lm_head_upload(pl, ps, n, pr, pf, L, max_chunk, override, tok_cap, seg_cap,
                                  req_cap, staging, device, total * 4, info, nullptr, 0,
                                  nullptr);
  else
    rc = lora_plan_upload(pl, ps, n, pr, pf, L, decode, max_chunk, override, tok_cap, seg_cap,
                          req_cap, staging, device, total * 4, info, nullptr, 0, nullptr);
  std::ostringstream out;
  out << rc;
  put(out, info, 6);
  put(out, staging, total);
  std::cout << out.str() << '\n';
  std::free(staging);
  std::free(device);
  std::free(pl);
  std::free(ps);
  std::free(pr);
  std::free(pf);
}

// lora_plan_upload_embedding over stand-in device buffers: the staging
// buffer as U, and whether the one-launch form was taken, with the slots
// and ranks it was given.
void cmd_upload_embedding(std::istringstream& in) {
  alignas(256) static int64_t ids[4096];       // stand-ins for device tensors (never read)
  alignas(256) static uint16_t emb_a[1 << 12];
  alignas(256) static uint16_t emb_out[1 << 12];
  int decode, max_chunk, L, seg_cap, req_cap, has_lens, n, R;
  int64_t tok_cap;
  in >> decode >> max_chunk >> L >> tok_cap >> seg_cap >> req_cap >> has_lens >> n;
  std::vector<int32_t> lens = has_lens ? read_ints(in, n) : std::vector<int32_t>();
  std::vector<int32_t> slots = read_ints(in, n);
  std::vector<int32_t> ranks = read_ints(in, L);
  std::vector<int32_t> sbits = read_ints(in, L);
  in >> R;
  std::vector<float> scal(static_cast<size_t>(L));
  std::memcpy(scal.data(), sbits.data(), sizeof(float) * L);
  const int64_t total = lora_plan_layout(tok_cap, seg_cap, req_cap, L, nullptr);
  int32_t* staging = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * total));
  std::memset(staging, 0xff, sizeof(int32_t) * total);
  int32_t* device = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * total));
  int32_t* pl = exact(lens);
  int32_t* ps = exact(slots);
  int32_t* pr = exact(ranks);
  float* pf = exact(scal);
  int32_t info[6] = {-1, -1, -1, -1, -1, -1};
  const int before = sgg::g_fused_embeds;
  const int rc = lora_plan_upload_embedding(pl, ps, n, pr, pf, L, decode, max_chunk, 0, tok_cap,
                                            seg_cap, req_cap, staging, device, total * 4, info,
                                            nullptr, 0, ids, emb_a, 1000, emb_out, R, R, 1000,
                                            nullptr);
  const bool fused = sgg::g_fused_embeds != before;
  std::ostringstream out;
  out << rc;
  put(out, info, 6);
  put(out, staging, total);
  const sgg::EmbedUploadParams& e = sgg::g_last_embed;
  out << " | " << (fused ? 1 : 0) << ' ' << (fused ? e.s : 0) << ' ' << (fused ? e.R : 0) << ' '
      << (fused ? e.n : 0);
  if (fused) {
    out << " |";
    for (int32_t t = 0; t < e.s; ++t) out << ' ' << static_cast<int>(e.slot[t]);
    put(out, e.rank, sgg::kEmbedUploadMaxLoras);
  }
  std::cout << out.str() << '\n';
  std::free(staging);
  std::free(device);
  std::free(pl);
  std::free(ps);
  std::free(pr);
  std::free(pf);
}

// Validation cases: every entry point with arguments its host checks reject,
// and with arguments it accepts (the stub launchers enqueue nothing).
void cmd_validate() {
  alignas(256) static uint16_t act[1 << 16];   // stand-ins for device tensors (never read)
  alignas(256) static uint16_t wts[1 << 16];
  alignas(256) static uint16_t outb[1 << 16];
  alignas(256) static char ws[1 << 22];
  alignas(16) static int32_t ind[3] = {0, 8, 16};
  alignas(16) static int32_t sl[2] = {0, 1};
  alignas(16) static int32_t perm[16];
  alignas(16) static int32_t ranks[2] = {8, 8};
  alignas(16) static float scal[2] = {1.f, 1.f};
  alignas(16) static int64_t ids[16];
  int32_t offs1[2] = {0, 256};
  int32_t offs3[4] = {0, 128, 192, 256};
  int32_t offs_bad[3] = {0, 200, 100};
  struct Case {
    const char* name;
    int rc;
  };
  std::vector<Case> cases;
  auto shrink = [&](const void* x, int64_t K, int32_t c, int32_t R, int64_t ldh, void* w,
                    int64_t wb) {
    return lora_shrink(x, K, wts, outb, ldh, 16, K, 2, c, R, ind, sl, 2, perm, ranks, 16, w, wb,
                       nullptr);
  };
  cases.push_back({"shrink_ok", shrink(act, 256, 1, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_null_x", shrink(nullptr, 256, 1, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_k0", shrink(act, 0, 1, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_c9", shrink(act, 256, 9, 8, 72, ws, sizeof(ws))});
  cases.push_back({"shrink_k_odd", shrink(act, 250, 1, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_ldh_small", shrink(act, 256, 2, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_misaligned", shrink(act + 1, 256, 1, 8, 8, ws, sizeof(ws))});
  cases.push_back({"shrink_empty_plan",
                   lora_shrink(act, 256, wts, outb, 8, 0, 256, 2, 1, 8, nullptr, nullptr, 0,
                               nullptr, nullptr, 16, nullptr, 0, nullptr)});
  auto expand = [&](const int32_t* offs, int32_t c, int32_t max_slice, int32_t R, int64_t N,
                    void* out) {
    return lora_expand(act, static_cast<int64_t>(c) * R, wts, N, out, 256, 16, 2, R, offs, c,
                       max_slice, ind, sl, 2, perm, ranks, scal, 16, nullptr);
  };
  cases.push_back({"expand_ok", expand(offs1, 1, 256, 8, 256, outb)});
  cases.push_back({"expand_stacked_ok", expand(offs3, 3, 128, 8, 256, outb)});
  cases.push_back({"expand_offsets_decrease", expand(offs_bad, 2, 200, 8, 256, outb)});
  cases.push_back({"expand_max_slice_small", expand(offs3, 3, 64, 8, 256, outb)});
  cases.push_back({"expand_rank_above_128", expand(offs1, 1, 256, 136, 256, outb)});
  cases.push_back({"expand_b_rows_short", expand(offs1, 1, 256, 8, 128, outb)});
  cases.push_back({"expand_null_base", expand(offs1, 1, 256, 8, 256, nullptr)});
  auto qkv = [&](int64_t wbytes) {
    return lora_qkv(act, 256, wts, wts, 256, outb, 256, 16, 256, 2, 8, offs3, 3, 128, ind, sl, 2,
                    perm, ranks, scal, 16, ws, wbytes, nullptr);
  };
  cases.push_back({"qkv_ok", qkv(sizeof(ws))});
  cases.push_back({"qkv_workspace_small", qkv(64)});
  cases.push_back({"workspace_sizes",
                   lora_qkv_workspace_bytes(16, 256, 3, 8, 2, 16) > 0 &&
                           lora_shrink_workspace_bytes(4096, 4096, 3, 16, 40, 128) >= 0
                       ? 0
                       : 1});
  auto emb = [&](int32_t extra, int64_t vocab) {
    return lora_a_embedding(ids, wts, 1000, outb, 8, 16, 2, 8, vocab, ind, sl, 2, perm, ranks,
                            extra, nullptr);
  };
  cases.push_back({"embedding_ok", emb(0, 1000)});
  cases.push_back({"embedding_extra_vocab", emb(1, 1000)});
  cases.push_back({"embedding_vocab_above_v", emb(0, 1001)});
  alignas(16) static int32_t dplan[1 << 12];
  alignas(16) static int32_t dinfo[8];
  alignas(16) static int32_t dslots[4] = {0, 1, 0, 1};
  cases.push_back({"plan_device_ok",
                   lora_plan_device(nullptr, dslots, 4, ranks, scal, 2, 1, 128, 0, 4, 4, 4, dplan,
                                    sizeof(dplan), dinfo, nullptr)});
  cases.push_back({"plan_device_too_many_loras",
                   lora_plan_device(nullptr, dslots, 4, ranks, scal, 2000, 1, 128, 0, 4, 4, 4,
                                    dplan, sizeof(dplan), dinfo, nullptr)});
  cases.push_back({"plan_device_buffer_small",
                   lora_plan_device(nullptr, dslots, 4, ranks, scal, 2, 1, 128, 0, 4, 4, 4, dplan,
                                    16, dinfo, nullptr)});
  alignas(16) static int32_t mind[3] = {0, 2, 4};
  alignas(16) static int32_t mtopk[8] = {0, 1, 1, 0, 0, 1, 1, 0};
  auto moe_plan = [&](int64_t tokens, int32_t experts, int64_t bytes, int32_t* plan) {
    return lora_moe_plan(mind, sl, 2, mtopk, tokens, 2, experts, ranks, scal, 2, 128, 16, plan,
                         bytes, dinfo, nullptr);
  };
  cases.push_back({"moe_plan_ok", moe_plan(4, 2, sizeof(dplan), dplan)});
  cases.push_back({"moe_plan_too_many_copies", moe_plan(4096, 2, sizeof(dplan), dplan)});
  cases.push_back({"moe_plan_too_many_virtual", moe_plan(4, 512, sizeof(dplan), dplan)});
  cases.push_back({"moe_plan_buffer_small", moe_plan(4, 2, 16, dplan)});
  cases.push_back({"moe_plan_null_plan", moe_plan(4, 2, sizeof(dplan), nullptr)});
  for (const Case& c : cases) std::cout << c.name << ' ' << c.rc << '\n';
  std::cout << "launches " << sgg::g_launches << '\n';
  std::cout << "end\n";
}

}  // namespace

int main() {
  std::ios::sync_with_stdio(false);
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    char cmd = 0;
    in >> cmd;
    if (cmd == 'P') cmd_plan(in, false);
    else if (cmd == 'H') cmd_plan(in, true);
    else if (cmd == 'U') cmd_upload(in);
    else if (cmd == 'E') cmd_upload_embedding(in);
    else if (cmd == 'V') cmd_validate();
    else if (cmd != 0) std::cout << "unknown " << cmd << '\n';
  }
  std::cout.flush();
  return 0;
}
