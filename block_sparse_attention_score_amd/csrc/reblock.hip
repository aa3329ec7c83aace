// Spark-Reblock partition (Spark-H3 page, section "Spark-Attnが変えるもの", Spark-Reblock bullet).
// Not built yet: the workspace size is 0, so spark_attn_reblock reports SPARK_ATTN_UNSUPPORTED.
#include "kernels.hpp"

namespace spark {

size_t reblock_workspace_bytes(const LaunchCtx&) { return 0; }

void launch_reblock(const LaunchCtx&, const void*, const void*, int32_t*, void*) {}

}  // namespace spark
