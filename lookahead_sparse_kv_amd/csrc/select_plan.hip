// select_plan.hip -- the select, plan and fused select + plan kernels with
// 256 threads per row (select_plan_impl.h); rows wider than kWideRowMinWidth
// blocks go to the 1024-thread build of the same code (select_plan_wide.hip).
#include "select_plan_impl.h"
