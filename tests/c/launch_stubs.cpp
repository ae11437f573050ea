// Host-only stand-ins for the kernel launchers of fb_kernels.hip and the four
// HIP runtime calls fb_api.cpp makes, so the whole host layer (validation,
// split planning, launch arguments) runs on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Each stub checks what the real launcher relies
// on: a dispatch's work-item count stays inside 32 bits, the attention grid
// covers its work items, and the split plan's partials fit the workspace the
// host layer asked for.  A violated check aborts the program.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "fb_internal.h"

static void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch check failed: %s\n", what);
    abort();
  }
}

static const int64_t kWorkItemLimit = (int64_t)1 << 32;
static const int64_t kCappedBlocks = (int64_t)1 << 20;

static int64_t capped(int64_t blocks) { return blocks < kCappedBlocks ? blocks : kCappedBlocks; }

extern "C" {
long long g_launches = 0;
}

namespace fb {

int launch_attn(const AttnArgs& a, int dtype, int head_dim, int cfg, bool partial, void* stream) {
  (void)stream;
  ++g_launches;
  require(dtype == 0 || dtype == kDtypeBf16, "dtype");
  require(head_dim == 64 || head_dim == 128, "head_dim");
  require(a.n_work >= 0 && a.grid >= a.n_work && a.grid % 8 == 0 && a.grid - a.n_work < 8, "grid covers work");
  const int threads = dtype == 0 ? 256 : 64 * 8;   // at most 8 waves per workgroup
  require((int64_t)a.grid * threads < kWorkItemLimit, "attention grid work items");
  require(a.rows == a.G * a.Lb && a.G * a.Hkv == a.Hq, "rows and heads");
  if (dtype != 0) require(cfg_info(cfg).rows > 0, "configuration");
  if (partial) {
    require(a.offsets != nullptr && a.part_o != nullptr && a.part_lse != nullptr, "partial outputs");
    require(a.split_tiles >= 1 && a.row_tiles >= 1, "split plan");
  } else {
    require(a.o != nullptr, "block output");
  }
  return 0;
}

int launch_combine(const CombineArgs& c, int64_t rows, void* stream) {
  (void)stream;
  ++g_launches;
  require(rows == (int64_t)c.B * c.Hq * c.Lb, "combine rows");
  require(capped((rows + 3) / 4) * 256 < kWorkItemLimit, "combine work items");
  require(c.total_splits >= 0, "combine splits");
  return 0;
}

int launch_merge(int64_t rows, int32_t head_dim, const float* oa, const float* la, const float* ob, const float* lb,
                 float* o, float* lse, void* stream) {
  (void)head_dim, (void)oa, (void)la, (void)ob, (void)lb, (void)o, (void)lse, (void)stream;
  ++g_launches;
  require(capped((rows + 3) / 4) * 256 < kWorkItemLimit, "merge work items");
  return 0;
}

int launch_tau(const TauArgs& t, void* stream) {
  (void)stream;
  ++g_launches;
  require(capped(((int64_t)t.B * t.Lb + 3) / 4) * 256 < kWorkItemLimit, "tau flag work items");
  require((int64_t)t.B * 256 < kWorkItemLimit, "tau finalize work items");
  return 0;
}

int launch_append(const AppendArgs& a, void* stream) {
  (void)stream;
  ++g_launches;
  const int64_t n = 2LL * a.B * a.Lb * a.Hkv * (a.D * a.esize / 16);
  require(capped((n + 255) / 256) * 256 < kWorkItemLimit, "append work items");
  return 0;
}

int launch_pool(const SelectArgs& a, void* stream) {
  (void)stream;
  ++g_launches;
  const int64_t waves = (int64_t)a.B * (a.max_chunks - a.first_chunk) * a.Hkv;
  require(capped((waves + 3) / 4) * 256 < kWorkItemLimit, "pool work items");
  return 0;
}

int launch_select_pooled(const SelectArgs& a, void* stream) {
  (void)stream;
  ++g_launches;
  const int64_t tiles = (int64_t)a.B * a.Hkv * ((a.max_chunks + 63) / 64);
  require(tiles * 256 < kWorkItemLimit, "score work items");
  require((int64_t)a.B * a.Hkv * 1024 < kWorkItemLimit, "top-k work items");
  require(a.max_chunks <= kMaxSelectChunks && a.k >= 1, "top-k capacity");
  return 0;
}

int launch_gamma(const GammaArgs& g, void* stream) {
  (void)stream;
  ++g_launches;
  require((int64_t)g.B * g.Hkv * 1024 < kWorkItemLimit, "gamma work items");
  return 0;
}

int launch_nan_scan(const float* x, int64_t n, int32_t* flag, bool clear, void* stream) {
  (void)x, (void)n, (void)flag, (void)clear, (void)stream;
  ++g_launches;
  return 0;
}

int launch_chunk_check(const int32_t* list, const int64_t* offsets, int32_t B, int32_t Hkv, int32_t k,
                       int32_t chunk_len, int32_t* flag, void* stream) {
  (void)list, (void)offsets, (void)B, (void)Hkv, (void)k, (void)chunk_len, (void)flag, (void)stream;
  ++g_launches;
  return 0;
}

int launch_unit_plan(const UnitPlanArgs& u, void* stream) {
  (void)stream;
  ++g_launches;
  require(u.mask != nullptr && u.plan != nullptr && u.row_tiles >= 1 && u.min_split >= 1 && u.cap >= 0,
          "unit plan arguments");
  require((int64_t)u.B * u.Hkv <= ((int64_t)1 << 21), "unit plan pairs");
  return 0;
}

int noalloc_scratch(void** ptr) {
  *ptr = (void*)(uintptr_t)0x40000000;   // an aligned stand-in address, never dereferenced on the host
  return 0;
}

}  // namespace fb

// the HIP runtime calls of the host layer (only on the FB_DEBUG and error paths)
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t sizeBytes, hipMemcpyKind kind, hipStream_t stream) {
  (void)src, (void)kind, (void)stream;
  for (size_t i = 0; i < sizeBytes; ++i) ((char*)dst)[i] = 0;   // "no problem found"
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t stream) {
  (void)stream;
  return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t stream, hipStreamCaptureStatus* pCaptureStatus) {
  (void)stream;
  *pCaptureStatus = hipStreamCaptureStatusNone;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t hipError) {
  (void)hipError;
  return "stub";
}
