// K-tail kernels of table row 4 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(4, Fast4)
