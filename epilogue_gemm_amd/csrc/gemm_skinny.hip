// gemm_skinny.hip -- the decode-shape kernel's configuration table, the
// shapes each configuration takes, the plan's choice among them and the
// dispatch to the per-format units (the kernel: gemm_skinny.hpp).
#include "kernels.hpp"

namespace ge {
namespace {

// Configuration indices are part of the ABI (gemm_epi_plan_select); the
// plan's preference order is kSkinnyPref below.  LDS: A's ring P x 32 rows
// x 2 KC bytes, B's P x CW columns x 2 KC bytes.
const SkinnyConfig kSkinny[] = {
    {8, 5, 256, "skinny_32n_8w_5x256k", false, 32},  // 80 + 80 KiB: four chunks of 512-byte row segments in flight
    {8, 4, 256, "skinny_32n_8w_4x256k", false, 32},  // 64 + 64 KiB
    {4, 4, 256, "skinny_32n_4w_4x256k", false, 32},  // 64 + 64 KiB, fewer waves
    {4, 8, 128, "skinny_32n_4w_8x128k", false, 32},  // 64 + 64 KiB, 256-byte row segments, seven chunks in flight
    {4, 2, 256, "skinny_32n_4w_2x256k", false, 32},  // 32 + 32 KiB: K down to 512
    {2, 2, 128, "skinny_32n_2w_2x128k", false, 32},  // 16 + 16 KiB: K down to 256
    // B row-major: 64-byte row pieces of 32 columns, transposing LDS reads
    {8, 5, 256, "skinny_rowb_32n_8w_5x256k", true, 32},
    {4, 8, 128, "skinny_rowb_32n_4w_8x128k", true, 32},
    {2, 2, 128, "skinny_rowb_32n_2w_2x128k", true, 32},
    // B row-major, 64 columns: 128-byte row pieces; 96 + 48 KiB
    {8, 6, 128, "skinny_rowb_64n_8w_6x128k", true, 64},
};

}  // namespace

int skinny_num_configs() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const SkinnyConfig& skinny_config(int cfg) { return kSkinny[cfg]; }

bool skinny_supports(int cfg, const Problem& p) {
  if (cfg < 0 || cfg >= skinny_num_configs()) return false;
  // K a multiple of 8 (a partial chunk is padded to KC with zeros) and at
  // least one chunk per ring slot; rows 16-byte aligned (leading dimensions
  // multiples of 8); 32 rows of B and all of A must be addressable by one
  // buffer resource
  // (row-major B: the workgroup's buffer spans all K rows, K ldb 2 < 2^32)
  // A column-major B takes any N and any ldc: with N % 8 != 0 or N < 32
  // the last workgroup is not shifted back but masked past N, and a quad of
  // outputs that reaches past N, or rows of C not 4-element aligned, are
  // stored element by element.  A row-major B keeps N % 8 = 0, N >= the
  // workgroup's columns and 16-byte rows of C.
  const SkinnyConfig& c = kSkinny[cfg];
  const bool b_ok = c.brow ? p.lb == GEMM_EPI_ROW_MAJOR && p.K * p.ldb * 2 < ((int64_t)1 << 32) && p.N >= c.cols &&
                                 p.N % 8 == 0 && p.ldc % 8 == 0
                           : p.lb == GEMM_EPI_COL_MAJOR && 32 * p.ldb * 2 < ((int64_t)1 << 31);
  return p.M >= 1 && p.M <= 32 && p.la == GEMM_EPI_ROW_MAJOR && b_ok && p.N >= 1 && p.K % 8 == 0 &&
         (p.K + c.kc - 1) / c.kc >= c.stages && p.lda % 8 == 0 && p.ldb % 8 == 0 && p.M * p.lda * 2 < ((int64_t)1 << 32);
}

int skinny_split(int cfg, const Problem& p) {
  const SkinnyConfig& c = kSkinny[cfg];
  const int64_t nblocks = (p.N + c.cols - 1) / c.cols, chunks = (p.K + c.kc - 1) / c.kc;
  int s = 1;
  while (nblocks * s < 256 && chunks % (2 * s) == 0 && chunks / (2 * s) >= c.stages && s < 16) s *= 2;
  return s;
}

// In order of preference (a row-major B prefers 64-column workgroups:
// 32 x 8192 x 8192 bf16 43.0 us against 46.1 us for 32 columns): the first
// configuration whose chunk divides K; else the first one that pads the
// first, partial chunk.
static const int kSkinnyPref[] = {0, 1, 2, 3, 4, 5, 9, 6, 7, 8};
static_assert(sizeof(kSkinnyPref) / sizeof(kSkinnyPref[0]) == sizeof(kSkinny) / sizeof(kSkinny[0]), "preference");

int skinny_choose(const Problem& p) {
  for (int c : kSkinnyPref)
    if (p.K % kSkinny[c].kc == 0 && skinny_supports(c, p)) return c;
  for (int c : kSkinnyPref)
    if (skinny_supports(c, p)) return c;
  return -1;
}

LaunchFn skinny_launcher(int cfg, const Problem& p) {
  if (p.in_dt == GEMM_EPI_F16) {
    if (p.out_dt == GEMM_EPI_F16) return skinny_launcher_f16_f16(cfg, p.epi);
    if (p.out_dt == GEMM_EPI_F32) return skinny_launcher_f16_f32(cfg, p.epi);
    if (p.out_dt == GEMM_EPI_FP8_E4M3) return skinny_launcher_f16_fp8(cfg, p.epi);
  } else if (p.in_dt == GEMM_EPI_BF16) {
    if (p.out_dt == GEMM_EPI_BF16) return skinny_launcher_bf16_bf16(cfg, p.epi);
    if (p.out_dt == GEMM_EPI_F32) return skinny_launcher_bf16_f32(cfg, p.epi);
    if (p.out_dt == GEMM_EPI_FP8_E4M3) return skinny_launcher_bf16_fp8(cfg, p.epi);
  }
  return nullptr;
}

}  // namespace ge
