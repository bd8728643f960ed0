// Host-only driver for the argument checks (built with g++ and sanitizers, no GPU).
// Forces every status code of every entry point's check from the host and checks
// the workspace layout; exits non-zero on the first mismatch.
#include <cstdio>
#include <cstdlib>

#include "../config.h"
#include "../validate.h"

using namespace moe;

static int failures = 0;
static void expect(const char* what, moe_status got, moe_status want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, static_cast<int>(got), static_cast<int>(want));
    ++failures;
  }
}

int main() {
  alignas(256) static unsigned char buf[4096];
  const void* p = buf;                 // 256-aligned stand-in pointer
  const void* odd = buf + 1;           // misaligned
  const void* p4 = buf + 4;            // 4- but not 16-aligned

  // route
  expect("route ok", check_route(p, 16, 256, 6, p, p), MOE_OK);
  expect("route T=0 nulls", check_route(nullptr, 0, 256, 6, nullptr, nullptr), MOE_OK);
  expect("route T<0", check_route(p, -1, 256, 6, p, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route k=0", check_route(p, 16, 256, 0, p, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route k>E", check_route(p, 16, 4, 5, p, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route E=0", check_route(p, 16, 0, 1, p, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route E>1024", check_route(p, 16, 1025, 6, p, p), MOE_ERR_UNSUPPORTED);
  expect("route k>8", check_route(p, 16, 256, 9, p, p), MOE_ERR_UNSUPPORTED);
  expect("route T*k overflow", check_route(p, (int64_t)1 << 31, 256, 6, p, p), MOE_ERR_UNSUPPORTED);
  expect("route null logits", check_route(nullptr, 16, 256, 6, p, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route null ids", check_route(p, 16, 256, 6, nullptr, p), MOE_ERR_INVALID_ARGUMENT);
  expect("route misaligned", check_route(odd, 16, 256, 6, p, p), MOE_ERR_MISALIGNED);

  // bitmatrix
  expect("bm ok", check_bitmatrix(p, 16, 256, 6, p), MOE_OK);
  expect("bm null", check_bitmatrix(p, 16, 256, 6, nullptr), MOE_ERR_INVALID_ARGUMENT);
  expect("bm misaligned", check_bitmatrix(p, 16, 256, 6, odd), MOE_ERR_MISALIGNED);
  expect("bm T=0", check_bitmatrix(nullptr, 0, 256, 6, nullptr), MOE_OK);

  // offsets
  WsLayout L;
  expect("layout", workspace_layout(8191, 256, 6, 4096, 2048, &L), MOE_OK);
  if (L.n_blocks != 16 || L.offsets_bytes != 16 * 256 * 4) { std::printf("FAIL offsets layout\n"); ++failures; }
  if (L.tile_bound != (49146 + (kFfnMinTileRows - 1) * 256) / kFfnMinTileRows) {
    std::printf("FAIL tile bound\n"); ++failures;
  }
  // decode sizes (T k < E, K of 2048 / 4096): 1-row tiles on the GEMV kernels
  WsLayout G;
  expect("layout gemv", workspace_layout(8, 256, 6, 4096, 2048, &G), MOE_OK);
  if (ffn_tile_rows(8, 256, 6, 4096, 2048) != kFfnGemvTileRows || G.tile_bound != 48) {
    std::printf("FAIL gemv tile rule / bound\n"); ++failures;
  }
  if (ffn_tile_rows(8, 256, 6, 256, 128) != 16 || ffn_tile_rows(43, 256, 6, 4096, 2048) != 16) {
    std::printf("FAIL gemv tile rule limits\n"); ++failures;
  }
  // ffn_tile_bound against the exact tile count of random and extreme row counts
  {
    unsigned rng = 12345u;
    auto next = [&]() { rng = rng * 1664525u + 1013904223u; return rng >> 8; };
    const int sizes[] = {2, 16, 32, 80, 128};
    for (int trial = 0; trial < 2000; ++trial) {
      const int E = 1 + static_cast<int>(next() % 300);
      const int R = sizes[trial % 5];
      static int c[300];
      int64_t n = 0, tiles = 0;
      for (int e = 0; e < E; ++e) {
        const unsigned kind = trial % 4;   // sparse, 1 mod R, skewed, uniform
        c[e] = kind == 0 ? (next() % 5 == 0 ? static_cast<int>(next() % 4) : 0)
             : kind == 1 ? static_cast<int>(R * (next() % 3) + 1)
             : kind == 2 ? (e == 0 ? static_cast<int>(next() % 5000) : static_cast<int>(next() % 3))
                         : static_cast<int>(next() % 200);
        n += c[e];
        tiles += (c[e] + R - 1) / R;
      }
      if (tiles > ffn_tile_bound(n, E, R)) {
        std::printf("FAIL tile bound trial %d: %lld tiles > %lld\n", trial,
                    static_cast<long long>(tiles), static_cast<long long>(ffn_tile_bound(n, E, R)));
        ++failures;
        break;
      }
    }
  }
  if (L.ffn_plan_offset < (size_t)49146 * 2048 * 2 || L.total < L.ffn_bytes || L.total < L.offsets_bytes) {
    std::printf("FAIL ffn layout\n"); ++failures;
  }
  expect("offs ok", check_offsets(p, p, 16, 256, 6, p, p, p, p, p, L.total), MOE_OK);
  expect("offs small ws", check_offsets(p, p, 1025, 256, 6, p, p, p, p, p, 256 * 4), MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("offs ws misaligned", check_offsets(p, p, 16, 256, 6, p, p, p, p, p4, 1 << 20), MOE_ERR_MISALIGNED);
  expect("offs null gather", check_offsets(p, p, 16, 256, 6, p, p, nullptr, p, p, 1 << 20), MOE_ERR_INVALID_ARGUMENT);
  expect("offs T=0", check_offsets(nullptr, nullptr, 0, 256, 6, p, p, nullptr, nullptr, nullptr, 0), MOE_OK);
  expect("offs T=0 null counts", check_offsets(nullptr, nullptr, 0, 256, 6, nullptr, p, nullptr, nullptr, nullptr, 0), MOE_ERR_INVALID_ARGUMENT);

  // ffn
  WsLayout F;
  workspace_layout(16, 256, 6, 256, 128, &F);
  expect("ffn ok", check_ffn(p, 16, 256, 128, 256, 6, p, p, p, p, p, p, p, p, p, F.ffn_bytes), MOE_OK);
  expect("ffn H%128", check_ffn(p, 16, 192, 128, 256, 6, p, p, p, p, p, p, p, p, p, 1 << 30), MOE_ERR_UNSUPPORTED);
  expect("ffn I%128", check_ffn(p, 16, 256, 64, 256, 6, p, p, p, p, p, p, p, p, p, 1 << 30), MOE_ERR_UNSUPPORTED);
  expect("ffn H=0", check_ffn(p, 16, 0, 128, 256, 6, p, p, p, p, p, p, p, p, p, 1 << 30), MOE_ERR_INVALID_ARGUMENT);
  expect("ffn small ws", check_ffn(p, 16, 256, 128, 256, 6, p, p, p, p, p, p, p, p, p, F.ffn_bytes - 1), MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("ffn x misaligned", check_ffn(p4, 16, 256, 128, 256, 6, p, p, p, p, p, p, p, p, p, F.ffn_bytes), MOE_ERR_MISALIGNED);
  expect("ffn w1 misaligned", check_ffn(p, 16, 256, 128, 256, 6, p4, p, p, p, p, p, p, p, p, F.ffn_bytes), MOE_ERR_MISALIGNED);
  expect("ffn w1 scales misaligned", check_ffn(p, 16, 256, 128, 256, 6, p, p4, p, p, p, p, p, p, p, F.ffn_bytes), MOE_ERR_MISALIGNED);
  expect("ffn w2 scales misaligned", check_ffn(p, 16, 256, 128, 256, 6, p, p, p, p4, p, p, p, p, p, F.ffn_bytes), MOE_ERR_MISALIGNED);
  expect("ffn null w2s", check_ffn(p, 16, 256, 128, 256, 6, p, p, p, nullptr, p, p, p, p, p, F.ffn_bytes), MOE_ERR_INVALID_ARGUMENT);
  expect("ffn T=0", check_ffn(nullptr, 0, 256, 128, 256, 6, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0), MOE_OK);

  // combine
  expect("comb ok", check_combine(p, p, p, 16, 256, 6, p), MOE_OK);
  expect("comb H%8", check_combine(p, p, p, 16, 260, 6, p), MOE_ERR_UNSUPPORTED);
  expect("comb k=0", check_combine(p, p, p, 16, 256, 0, p), MOE_ERR_INVALID_ARGUMENT);
  expect("comb y misaligned", check_combine(p, p, p, 16, 256, 6, p4), MOE_ERR_MISALIGNED);
  expect("comb null", check_combine(p, nullptr, p, 16, 256, 6, p), MOE_ERR_INVALID_ARGUMENT);
  expect("comb T=0", check_combine(nullptr, nullptr, nullptr, 0, 256, 6, nullptr), MOE_OK);

  if (failures) return 1;
  std::printf("validate_check ok\n");
  return 0;
}
