// select_plan_wide.hip -- the select, plan and fused select + plan kernels
// built with 1024 threads per row (namespace oasis::wide), for rows of more
// than kWideRowMinWidth blocks: four times the lanes for the row's key loads,
// histogram passes and compaction, on the few CUs such rows occupy.
#define OASIS_ROW_WIDE 1
#include "select_plan_impl.h"
