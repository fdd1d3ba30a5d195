// Host-only stand-ins for the kernel launchers, linked with the C-ABI
// validation layer (api.cpp) in the sanitizer build: a call that passes
// validation lands here, counts itself and returns success without touching
// any pointer, so AddressSanitizer and UBSan see only the host code.
#include "../../sparse_paged_mla_amd/csrc/launch.h"

namespace {
int g_launches = 0;
alignas(256) unsigned char g_fake_scratch[256];  // stands in for the static device workspace; never touched
}

namespace spmla {
int launch_indexer(const IndexerArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_topk(const TopkArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_decode(const DecodeArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_merge(const MergeArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_cache_append(const AppendArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_page_check(const PageCheckArgs&, hipStream_t) { return ++g_launches, 0; }
int launch_mq_expand(const MqExpandArgs&, hipStream_t) { return ++g_launches, 0; }
int topk_scratch(void** ptr) { return *ptr = g_fake_scratch, 0; }
}  // namespace spmla

extern "C" int spmla_stub_launches(void) { return g_launches; }
