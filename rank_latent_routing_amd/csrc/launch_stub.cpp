// Host-only stand-ins for the kernel launchers, linked with api.cpp and
// plan.cpp into libflare_host.so, a build of the C ABI with no device code.
// The CPU tests call every entry point through it, so an argument-check bug
// can never hand a bad pointer to a real kernel.  Each stand-in records the
// launch and returns a status the test chooses (hipSuccess by default), so a
// test can check that a failing launch becomes FLARE_E_HIP.  The stand-ins
// also record the device ranges a launch would write into the caller's
// workspace (split partials, swizzled weights, projection outputs), so a test
// can check that the workspace carving stays inside the workspace and that
// buffers live at the same time do not overlap.
#include <cstring>

#include "launch.hpp"

namespace {

enum RangeTag {
  kEncPartO = 1,   // encoder split outputs (written)
  kEncPartL = 2,   // encoder split normalisers (written)
  kBwdDq = 3,      // backward dQ split partials (written)
  kBwdDz = 4,      // backward dZ split partials (written)
  kSumPart = 5,    // split partials summed (read)
  kSwizzled = 6,   // swizzled projection weights (written)
  kGemmOut = 7,    // projection outputs (written)
  kEncK = 8,       // encoder K rows (read)
  kEncV = 9,       // encoder V rows (read)
  kWoLat = 10,     // fused output projection: prepared latent operands (written)
  kWoT = 11,       // fused output projection: prepared W_O^T (written)
  kDecZPart = 12,  // decoder: the encoder's split results, merged into Z while staged (read)
};

struct Range {
  unsigned long long addr, bytes;
  long launch;
  int tag, pad;
};

constexpr int kMaxRanges = 256;
int g_status = 0;
long g_launches = 0;
char g_last[64] = "";
Range g_ranges[kMaxRanges];
int g_nranges = 0;

hipError_t record(const char* name) {
  ++g_launches;
  std::strncpy(g_last, name, sizeof(g_last) - 1);
  return static_cast<hipError_t>(g_status);
}

void add_range(const void* p, unsigned long long bytes, int tag) {
  if (p == nullptr || g_nranges == kMaxRanges) return;
  g_ranges[g_nranges++] = Range{reinterpret_cast<unsigned long long>(p), bytes, g_launches, tag, 0};
}

// Bytes spanned by a [B, H, L, D] view with the given strides (last element + 1).
unsigned long long view_span(const flare::View& v, int B, int H, int64_t L, int D) {
  const int64_t esz = v.is_f32 ? 4 : 2;
  const int64_t last = (int64_t)(B - 1) * v.sb + (int64_t)(H - 1) * v.sh + (L - 1) * v.sl + D;
  return (unsigned long long)(last * esz);
}

}  // namespace

namespace flare {

hipError_t launch_encode_bf16(const EncodeParams& p, int D, int B, int, int, hipStream_t) {
  const unsigned long long parts = (unsigned long long)B * p.H * p.S * p.M;
  add_range(p.part_o, parts * D * 4, kEncPartO);
  add_range(p.part_l, parts * 4, kEncPartL);
  add_range(p.k.data, view_span(p.k, B, p.H, p.N, D), kEncK);
  add_range(p.v.data, view_span(p.v, B, p.H, p.N, D), kEncV);
  return record("encode_bf16");
}
hipError_t launch_encode_f32(const EncodeParams& p, int D, int B, hipStream_t s) {
  const hipError_t e = launch_encode_bf16(p, D, B, 0, 0, s);
  std::strncpy(g_last, "encode_f32", sizeof(g_last) - 1);
  return e;
}
hipError_t launch_merge(const MergeParams&, int, hipStream_t) { return record("merge"); }
hipError_t launch_decode_bf16(const DecodeParams& p, int D, int B, hipStream_t) {
  if (p.zm_part_o) {
    const unsigned long long zparts = (unsigned long long)B * p.H * p.zm_S * p.M;
    add_range(p.zm_part_o, zparts * D * 4, kDecZPart);
    add_range(p.zm_part_l, zparts * 4, kDecZPart);
  }
  return record("decode_bf16");
}
hipError_t launch_decode_f32(const DecodeParams&, int, int, hipStream_t) { return record("decode_f32"); }
hipError_t launch_tok_bwd(const TokBwdParams&, int, int, bool, hipStream_t) { return record("tok_bwd"); }
hipError_t launch_lat_bwd(const LatBwdParams& p, int D, int B, bool, hipStream_t) {
  const unsigned long long parts = (unsigned long long)B * p.H * p.S * p.M * D * 4;
  add_range(p.dq_part, parts, kBwdDq);
  add_range(p.dz_part, parts, kBwdDz);
  return record("lat_bwd");
}
hipError_t launch_tok_pair(const TokPairParams&, int, int, hipStream_t) { return record("tok_pair"); }
hipError_t launch_sum_splits(const float* part, float*, int B, int H, int S, int64_t MD, bool, float, int,
                             hipStream_t) {
  add_range(part, (unsigned long long)B * H * S * MD * 4, kSumPart);
  return record("sum_splits");
}
hipError_t launch_swizzle_weights(const SwizzleParams& p, int n, hipStream_t) {
  for (int i = 0; i < n; ++i) add_range(p.wsw[i], (unsigned long long)p.Cin * p.Cout * 2, kSwizzled);
  return record("swizzle_weights");
}
hipError_t launch_decode_wo(const DecodeWoParams& p, int B, const void*, hipStream_t) {
  add_range(p.lat_ops, (unsigned long long)B * p.H * ((p.M + 31) / 32) * 4096, kWoLat);
  add_range(p.wt, (unsigned long long)(32 * p.H) * (32 * p.H) * 2, kWoT);
  return record("decode_wo");
}
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t) {
  for (int i = 0; i < p.n_proj; ++i) add_range(p.y[i], (unsigned long long)p.R * p.Cout * 2, kGemmOut);
  return record("gemm_bf16");
}

}  // namespace flare

extern "C" {
// Test hooks of the host-only build (not part of include/flare.h).
void flare_stub_set_launch_status(int status) { g_status = status; }
void flare_stub_reset(void) {
  g_status = 0;
  g_launches = 0;
  g_last[0] = 0;
  g_nranges = 0;
}
long flare_stub_launches(void) { return g_launches; }
const char* flare_stub_last_launch(void) { return g_last; }
// Copies up to max recorded ranges as (addr, bytes, launch index, tag)
// quadruples of 64-bit integers; returns how many were recorded.
int flare_stub_ranges(unsigned long long* out, int max) {
  const int n = g_nranges < max ? g_nranges : max;
  for (int i = 0; i < n; ++i) {
    out[4 * i + 0] = g_ranges[i].addr;
    out[4 * i + 1] = g_ranges[i].bytes;
    out[4 * i + 2] = (unsigned long long)g_ranges[i].launch;
    out[4 * i + 3] = (unsigned long long)g_ranges[i].tag;
  }
  return g_nranges;
}
}
